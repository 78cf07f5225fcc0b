// Device-side routing prologue shared by the dispatch and combine kernels.
//
// The receive buffer of a set holds num_experts * max_tokens message rows
// (rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, struct LLMoEBuffer, dispatch
// receive buffer); expert e owns rows [e * max_tokens, (e + 1) * max_tokens).
// A routed entry (t, k) goes to row e * max_tokens + slot(t, k), where
// slot(t, k) counts the earlier entries, in (t, k) order, that name the same
// expert. That is an exclusive prefix count per expert in ascending token
// order, which makes the slot order deterministic.
//
// A workgroup serves a tile of consecutive tokens [t0, t1) and computes the
// slots of all the tile's entries at once from the routing table itself (no
// workspace, no second launch; the table is a few tens of KiB and stays in
// L2):
//   slot(j) = (entries before the tile naming e)      an LDS histogram
//           + (tile entries before j naming e)        a rank in registers
// The histogram lives in the caller's LDS and covers hist_cap experts per
// pass (min(num_experts, kHistExperts), sized at launch, so a small expert
// count leaves LDS to other workgroups); more experts take more passes over
// the earlier entries. Loads are unconditional (indices
// clamped into the table, clamped lanes masked afterwards), so the compiler
// issues them back to back. A round of loads covers UNROLL loads per thread
// of VEC consecutive entries each (VEC = 4: 16-byte loads, for tables that
// are 16-byte aligned and a whole number of 4-entry vectors). Fewer load
// instructions per thread measured faster even where they take more
// rounds: 1 load of 4 entries per thread and round in the register-path
// dispatch, 2 in the combine; 8 loads of 4 entries in the dispatch of
// 64 MiB or more, whose batch of 1024 tokens of 8 picks then takes one
// round (each choice is measured where it is made).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "layout.h"

namespace llmoe {

constexpr int kWave = 64;
constexpr int kHistExperts = 4096;
constexpr int kMaxTileEntries = kWave;  // tokens per tile * topk: one wavefront's lanes
static_assert(kMaxTileEntries == kTileEntryLimit, "tile limits of route.h and kernels.h");

// Histogram entries of the routing prologue for num_experts experts.
__host__ __device__ constexpr int hist_cap_for(int num_experts) {
  return num_experts < kHistExperts ? (num_experts > 0 ? num_experts : 1) : kHistExperts;
}

struct RouteShared {
  int expert[kMaxTileEntries];  // idx of the tile's entries, tile order
  int slot[kMaxTileEntries];    // their slots, or -1 when masked
};

// Number of lanes below this one in its 16-lane row (DPP row) whose v
// equals this lane's, for row shifts S..15: each step compares v with the
// value S lanes lower (row_shr:S); a lane whose source lies outside the row
// sees -1, which no valid expert equals.
template <int S>
__device__ __forceinline__ int same_below_in_row(int v) {
  if constexpr (S == 16) {
    return 0;
  } else {
    const int o = __builtin_amdgcn_update_dpp(-1, v, 0x110 + S, 0xF, 0xF, false);
    return (o == v) + same_below_in_row<S + 1>(v);
  }
}

struct NoOverlap {
  __device__ void operator()() const {}
};

// VEC consecutive entries of the routing table, read by one load.
template <int VEC>
struct IdxVec;
template <>
struct IdxVec<1> {
  typedef int32_t type;
  __device__ static int at(type v, int) { return v; }
};
template <>
struct IdxVec<4> {
  typedef int32_t type __attribute__((ext_vector_type(4)));
  __device__ static int at(type v, int j) { return v[j]; }
};

// Mask of the lanes below this one in its wavefront.
__device__ __forceinline__ uint64_t lanes_below() {
  return (1ull << (threadIdx.x & (kWave - 1))) - 1ull;
}

// Wavefront-wide grouping by value: for each distinct value v >= 0 held by
// the active lanes, calls f(v, mask of lanes holding v) on every lane (the
// loop is uniform). The loop runs once per distinct value, without memory.
template <typename F>
__device__ __forceinline__ void for_each_distinct(int value, const F& f) {
  uint64_t left = __ballot(value >= 0);
  while (left) {
    const int leader = __builtin_ctzll(left);
    const int v = __builtin_amdgcn_readlane(value, leader);
    const uint64_t same = __ballot(value == v);
    f(v, same);
    left &= ~same;
  }
}

// All threads of the workgroup must call this (it contains barriers).
// On return rs.expert[j] and rs.slot[j] hold entry j = (t - t0) * topk + k
// of the tile for t0 <= t < t1. Requires (t1 - t0) * topk <= kMaxTileEntries;
// hist is an LDS array of hist_cap >= 1 ints.
//
// Every global load of the first pass (the tile's own entries and the first
// round of earlier entries) is issued before anything waits on one, so the
// prologue costs one memory round trip, not two. `issue()` runs right after
// them, so that the caller's own loads travel in the same round trip;
// `overlap()` runs once on every thread after the first pass's histogram,
// before a barrier that both results share (the dispatch builds its first
// LDS message there), and `ready()` on every thread right after that
// barrier, while wavefront 0 goes on to compute the slots.
//
// Slots within the tile: an entry's slot is the histogram count of its
// expert plus its rank among the tile's earlier entries naming the same
// expert. The tile's entries sit in wavefront 0's lanes. For 4-16 entries
// (one DPP row) the rank is 15 row shifts and compares, with no dependent
// loop; otherwise a register walk over the earlier lanes (shorter for 1-3).
//
// VEC = 4 requires idx to be 16-byte aligned and the table (num_tokens *
// topk entries) to be a multiple of 4 entries long: every vector that holds
// an entry before the tile then lies wholly inside the table.
//
// WAVE_SLOTS: every wavefront holds the tile's entries in its lanes 0..n-1
// and computes their slots itself, returned in those lanes (-1 when
// masked), so that no barrier follows the slot computation when one
// histogram pass covers the experts; rs.slot is still written (by
// wavefront 0) and is visible after the caller's next barrier. Otherwise
// the return value is meaningless and rs.slot is visible on return.
template <int VEC = 1, bool WAVE_SLOTS = false, int UNROLL = 8, typename Issue = NoOverlap,
          typename Overlap = NoOverlap, typename Ready = NoOverlap>
__device__ __forceinline__ int route_tile(const int32_t* __restrict__ idx, int t0, int t1,
                                           int topk, int num_experts, int max_tokens,
                                           RouteShared& rs, int* hist, int hist_cap,
                                           const Issue& issue = Issue(),
                                           const Overlap& overlap = Overlap(),
                                           const Ready& ready = Ready()) {
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int first = t0 * topk;         // entries before the tile: [0, first)
  const int n = (t1 - t0) * topk;      // the tile's entries: [first, first + n)
  constexpr int kUnroll = UNROLL;
  typedef typename IdxVec<VEC>::type Vec;
  const Vec* tab = reinterpret_cast<const Vec*>(idx);
  const int stride = nthreads * kUnroll * VEC;  // entries per round
  // at least one round: the first round's loads are then consumed on every
  // path, so nothing later has to wait for them behind its own stores
  const int rounds = first > stride ? (first + stride - 1) / stride : 1;  // uniform
  const int last = first > 0 ? (first - 1) / VEC : 0;  // the load holding entry first - 1

  // loads of the first round and of the tile's own entries (threads j < n;
  // for a tile of up to 64 entries they stay in wavefront 0's registers);
  // indices are clamped into the table so the loads are unconditional
  Vec v0[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int q = tid + u * nthreads;
    v0[u] = tab[q < last ? q : last];
  }
  // the tile's own entries: in wavefront 0's lanes (WAVE_SLOTS: every
  // wavefront's) 0..n-1
  const int lane = WAVE_SLOTS ? (tid & (kWave - 1)) : tid;
  const int own = idx[first + (lane < n ? lane : 0)];
  issue();
  const int mine = lane < n ? own : -1;

  // One histogram pass over experts [c0, c0 + width). The first pass is a
  // separate instance (first_pass is a compile-time flag) that also runs
  // the callbacks and ranks the tile, so that they run on every path
  // through it: no load they consume can look in flight afterwards, which
  // would make a later wait cover the stores issued in between.
  int rank = 0;  // wavefront 0 (WAVE_SLOTS: all): earlier lanes holding the same expert
  int wslot = -1;  // WAVE_SLOTS: lane j's slot
  const bool multi_pass = num_experts > hist_cap;  // uniform
  auto pass = [&](int c0, auto first_pass) {
    constexpr bool kFirst = decltype(first_pass)::value;
    const int width = num_experts - c0 < hist_cap ? num_experts - c0 : hist_cap;
    for (int i = tid; i < width; i += nthreads) hist[i] = 0;
    __syncthreads();
    for (int it = 0; it < rounds; ++it) {
      const int base = it * (stride / VEC) + tid;  // in loads
      Vec v[kUnroll];
      if (kFirst && it == 0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = v0[u];
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int q = base + u * nthreads;
          v[u] = tab[q < last ? q : last];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const int p = (base + u * nthreads) * VEC + j;
          const unsigned rel = (unsigned)IdxVec<VEC>::at(v[u], j) - (unsigned)c0;
          if (p < first && rel < (unsigned)width) atomicAdd(&hist[rel], 1);
        }
      }
    }
    if constexpr (kFirst) {
      if (tid < n) {
        rs.expert[tid] = mine;
        rs.slot[tid] = -1;
      }
      overlap();
    }
    __syncthreads();
    if constexpr (kFirst) {
      ready();
      if (WAVE_SLOTS || tid < kWave) {
        if (n > 3 && n <= 16)  // uniform
          rank = same_below_in_row<1>(mine);
        else
          for (int j = 0; j < n; ++j)
            rank += (j < lane) & (__builtin_amdgcn_readlane(mine, j) == mine);
      }
    }
    if (WAVE_SLOTS || tid < kWave) {
      const unsigned rel = (unsigned)mine - (unsigned)c0;
      if (lane < n && rel < (unsigned)width) {
        const int s = hist[rel] + rank;
        wslot = s < max_tokens ? s : -1;
        if (tid < kWave) rs.slot[tid] = wslot;
      }
    }
    // the next pass clears hist: every wavefront must be done reading it
    if (!WAVE_SLOTS || multi_pass) __syncthreads();
  };
  pass(0, std::true_type{});
  for (int c0 = hist_cap; c0 < num_experts; c0 += hist_cap)  // uniform
    pass(c0, std::false_type{});
  return wslot;
}

}  // namespace llmoe
