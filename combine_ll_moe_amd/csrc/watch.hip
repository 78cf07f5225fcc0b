// A concurrent reader of a dispatch's signal words, for tests of the
// publish order: the counts are raised only after the messages they count
// are visible at device scope (mscclpp.h, the put-then-signal contract above
// struct mscclppDevConn: the receiver reads data only after it has seen the
// signal). Run on another stream while the dispatch runs.
//
// Workgroup b owns the experts e = b, b + G, ... (G workgroups). Before it
// polls, it works out from the routing which token every one of its
// experts' slots will hold: slot j of expert e is the j-th routed entry, in
// (token, pick) order, that names e. Then, pass after pass, it
//   1. loads its experts' counts with acquire semantics at device scope,
//   2. for every expert whose count has risen above the rows it has found
//      complete so far, compares each of that expert's not-yet-complete
//      receive rows, whole (every byte, header included), with the message
//      of the slot's token (an array the caller supplies),
//   3. records a violation for every expert whose acquired count exceeds
//      its complete rows.
// A row once complete stays complete (nothing else writes it), so a pass
// re-reads only rows that were not yet complete, and passes stay short
// while the dispatch runs. A workgroup stops once its acquired counts add
// up to its experts' routed messages, or after max_passes passes, so every
// workgroup ends. A row written but not yet counted may or may not be
// found; only a count ahead of its rows is wrong.
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
  const uint8_t* messages;         // [num_tokens, msg_bytes]: message(t) as it must be written
  const int32_t* idx;              // int32 [num_tokens, topk]
  int num_tokens;
  int max_tokens;
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
constexpr int kWatchWaves = kWatchBlock / 64;
// routed entries of a watched dispatch, at most (a workgroup's rows are a
// subset of them)
constexpr int kWatchMaxEntries = 4096;

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(kWatchBlock) watch_kernel(const WatchParams P) {
  __shared__ int cnt[kOwned];             // messages owned expert i will receive
  __shared__ int first[kOwned + 1];       // running sum of cnt: i's first row in the walk
  __shared__ int pub[kOwned];             // count acquired in this pass
  __shared__ int found[kOwned];           // rows found complete so far
  __shared__ int rowtok[kWatchMaxEntries];  // token whose message row r must hold
  __shared__ int todo[kWatchMaxEntries];  // rows to compare in this pass
  __shared__ uint8_t done[kWatchMaxEntries];
  __shared__ int ntodo;
  __shared__ long long total[2];
  __shared__ int violations;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid / 64;
  const int E = P.num_experts;
  const int K = P.topk;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int owned = b < E ? (E - 1 - b) / G + 1 : 0;  // experts b, b + G, ... below E
  const int entries = P.num_tokens * K;

  // the routing, staged in LDS (in `todo`, free until the passes start) and
  // walked in (token, pick) order once per owned expert: the token of every
  // slot (valid entries, slots below max_tokens). The walk is short, so the
  // watcher is polling before a dispatch held behind a brief spin starts.
  int* tab = todo;
  for (int j = tid; j < entries; j += kWatchBlock) tab[j] = P.idx[j];
  if (tid == 0) {
    total[0] = total[1] = 0;
    violations = 0;
  }
  __syncthreads();
  if (tid < owned) {
    const int e = b + tid * G;
    int c = 0;
    for (int j = 0; j < entries; ++j) c += tab[j] == e;
    cnt[tid] = c < P.max_tokens ? c : P.max_tokens;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < owned; ++i) {
      first[i] = run;
      run += cnt[i];
    }
    first[owned] = run;
  }
  __syncthreads();
  if (tid < owned) {
    const int e = b + tid * G;
    int c = 0;
    for (int j = 0; j < entries && c < cnt[tid]; ++j)
      if (tab[j] == e) rowtok[first[tid] + c++] = j / K;
    found[tid] = 0;
  }
  const int rows = first[owned];  // <= entries <= kWatchMaxEntries (host check)
  for (int r = tid; r < rows; r += kWatchBlock) done[r] = 0;
  __syncthreads();  // the table in `todo` is read everywhere before the passes reuse it
  const long long expected = rows;

  const uint32_t words = P.msg_bytes / 4;
  int partial = 0;
  int pass = 0;
  long long seen = 0;
  while (pass < P.max_passes) {  // uniform
    // 1. acquire the counts
    if (tid < owned) {
      const unsigned long long v = __hip_atomic_load(P.sig + b + tid * G, __ATOMIC_ACQUIRE,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      pub[tid] = (int)(uint32_t)v;
      atomicAdd(reinterpret_cast<unsigned long long*>(&total[pass & 1]), (unsigned long long)(uint32_t)v);
    }
    if (tid == 0) ntodo = 0;
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // 2. rows to compare: the not-yet-complete rows of experts whose count
    //    is above the rows found so far
    if (tid < owned && pub[tid] > found[tid])
      for (int r = first[tid]; r < first[tid + 1]; ++r)
        if (!done[r]) todo[atomicAdd(&ntodo, 1)] = r;
    __syncthreads();
    const int n = ntodo;
    for (int q = wave; q < n; q += kWatchWaves) {  // uniform per wavefront
      const int r = todo[q];
      int i = 0;
      while (i + 1 < owned && first[i + 1] <= r) ++i;
      const int e = b + i * G;
      const int j = r - first[i];
      const uint32_t* row = reinterpret_cast<const uint32_t*>(
          P.recv + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)j) * P.msg_bytes);
      const uint32_t* want = reinterpret_cast<const uint32_t*>(
          P.messages + (uint64_t)rowtok[r] * P.msg_bytes);
      bool same = true;
      for (uint32_t d = lane; d < words; d += 64) same = same && load_coherent(row + d) == want[d];
      if (__ballot(!same) == 0 && lane == 0) done[r] = 1;
    }
    __syncthreads();

    // 3. a count ahead of its complete rows is a violation
    if (tid < owned) {
      int f = 0;
      for (int r = first[tid]; r < first[tid + 1]; ++r) f += done[r];
      found[tid] = f;
      if (pub[tid] > f) atomicAdd(&violations, 1);
    }
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
                                 int num_experts, int topk, int dtype, int parity,
                                 const void* messages, const int32_t* topk_idx, int max_passes,
                                 long long* report, hipStream_t stream) {
  Layout L;
  if (parity != 0 && parity != 1) return LL_MOE_INVALID_ARGUMENT;
  if (!make_layout(max_tokens, hidden, num_experts, dtype, &L)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LL_MOE_INVALID_ARGUMENT;
  if (dtype == kBf16 && hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (topk < 1 || topk > num_experts || topk > LL_MOE_MAX_TOPK) return LL_MOE_INVALID_ARGUMENT;
  if (num_experts > kWatchMaxExperts || max_passes < 1) return LL_MOE_INVALID_ARGUMENT;
  if ((int64_t)num_tokens * topk > kWatchMaxEntries) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !report || !aligned(layout, 16) || !aligned(report, 8))
    return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens > 0 &&
      (!messages || !topk_idx || !aligned(messages, 4) || !aligned(topk_idx, 4)))
    return LL_MOE_INVALID_ARGUMENT;
  const uint8_t* base = static_cast<const uint8_t*>(layout);
  WatchParams p;
  p.sig = reinterpret_cast<const unsigned long long*>(base + L.sig_off(parity));
  p.recv = base + L.recv_off(parity);
  p.messages = static_cast<const uint8_t*>(messages);
  p.idx = topk_idx;
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.num_experts = num_experts;
  p.topk = topk;
  p.msg_bytes = (uint32_t)L.dispatch_msg;
  p.max_passes = max_passes;
  p.report = report;
  const int groups = num_experts < kWatchGroups ? num_experts : kWatchGroups;
  watch_kernel<<<groups, kWatchBlock, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? LL_MOE_SUCCESS : LL_MOE_HIP_ERROR;
}
