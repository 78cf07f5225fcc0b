// Two-phase combine: the expert side stages each output as a combine
// message and raises a flag per expert; the token side waits for the flags
// of its picks and folds the staged rows.
//
// What is computed (rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, struct
// LLMoEBuffer's combine buffers and flag, aliased by LLMoEBufferLayout's
// pointer table to the set's dispatch buffers; mscclpp.h, put-then-signal
// above struct mscclppDevConn; memra-engine src/tp_ar.rs, a fold ordered
// after the push and a bounded wait that leaves a refusal code):
//   expert side: for expert e and j < count_e, with t the header of receive
//     row e * max_tokens + j, staging row e * max_tokens + t := [int32 t |
//     expert output row e * max_tokens + j]; then the high half of signal
//     word e rises by the rows staged for e (count in the low half);
//   token side: once every routed pick's flag is up (high == low), the
//     fused combine's fma chain over the staging rows.
//
// Design on gfx950:
//  - Expert side. The work is the flattened (expert, slot) order of the
//    received messages, which only the counts describe: every workgroup
//    loads all counts and forms their exclusive prefix in LDS, then takes a
//    contiguous run of rows, 64 at a time. Lane l finds its row's expert by
//    binary search in the prefix and loads the row's header; then the
//    workgroup copies the rows one by one (the source row is 16-byte
//    aligned, the staging row starts at any 4-byte phase, and the phase is
//    only known once the header is back: the row's loads go out together
//    with the header load), next row's loads in flight while the current
//    row is stored: straight from registers with dword-aligned stores below
//    64 MiB of staged rows, through LDS with destination-aligned whole-line
//    stores above (mostly HBM-bound writes). Release as in the dispatch:
//    device-coherent stores, each wave waits for its own, a barrier, then
//    wave 0 adds per distinct expert the rows it staged to the flag with one
//    device-scope atomic on the word's high half.
//  - Token side. Workgroup 0 polls every expert's flag (relaxed
//    device-scope loads, at most max_spins rounds) and posts the outcome in
//    a caller-zeroed status word; every other workgroup looks at the flags
//    once and, if some are down, polls that one word, so that the waiting
//    adds almost no traffic to the signal words the expert side is raising.
//    Then work items of (tile of tokens, run of columns), as the
//    fused combine but with no routing prologue (a token's staging row for
//    pick k is e * max_tokens + t), over a grid of at most kRecvBlocks
//    workgroups that leaves a not-yet-started expert side room to run: the
//    fused combine's gather and fma chain over the staged payload, read
//    with device-coherent loads (4 bytes past the row start, so 4-byte
//    aligned 16-byte loads).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "expert.h"
#include "gather.h"
#include "kernels.h"
#include "message.h"
#include "route.h"

namespace llmoe {


// Rows at or above this many bytes go out with whole-cache-line lane
// mapping (mostly HBM-bound writes); smaller ones stay in the caches.
constexpr uint64_t kSendLineBytes = 64ull << 20;

// Staging through LDS with destination-aligned whole-line stores, for
// batches of kSendLineBytes or more (mostly HBM-bound writes).
__device__ __forceinline__ void stage_rows(const SendParams& P, uint32_t* pre, uint8_t* lds_msg,
                                           uint32_t msg_stride, int nbuf, uint32_t r0, uint32_t r1) {
  constexpr int kStage = 4;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int E = P.num_experts;
  const int chunks = P.hidden / 8;
  const uint32_t mc = P.comb_bytes;
  const u32x4* y = reinterpret_cast<const u32x4*>(P.y);
  auto msg_buffer = [&](int i) { return lds_msg + (nbuf == 2 ? (i & 1) : 0) * msg_stride; };

  for (uint32_t b0 = r0; b0 < r1; b0 += kWave) {
    const int n = r1 - b0 < (uint32_t)kWave ? (int)(r1 - b0) : kWave;
    // this lane's row of the batch: expert, slot and header
    const uint32_t r = b0 + (uint32_t)(lane < n ? lane : n - 1);
    const int e_l = expert_of_row(pre, E, r);
    const int j_l = (int)(r - pre[e_l]);
    const uint64_t src_l = (uint64_t)e_l * (uint64_t)P.max_tokens + (uint64_t)j_l;
    const int t_l = *reinterpret_cast<const int32_t*>(P.recv + src_l * P.msg_bytes);

    auto src_row = [&](int i) {
      const int e = __builtin_amdgcn_readlane(e_l, i);
      const int j = __builtin_amdgcn_readlane(j_l, i);
      return y + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)j) * (uint64_t)chunks;
    };
    u32x4 v[kStage];
    load_row<kStage>(v, src_row(0), chunks);
    for (int i = 0; i < n; ++i) {
      uint8_t* msg = msg_buffer(i);
      if (nbuf == 1 && i > 0) __syncthreads();  // the single buffer is still being read
      // message = [t | row]: the row's first kStage rounds from registers,
      // further rounds (hidden > kStage * 8 * blockDim) straight through
      const int t = __builtin_amdgcn_readlane(t_l, i);
      if (tid == 0) *reinterpret_cast<int32_t*>(msg) = t;
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int c = tid + u * kSendBlock;
        if (c < chunks) *reinterpret_cast<u32x4*>(msg + 4 + 16 * c) = v[u];
      }
      const u32x4* src = src_row(i);
      for (int c = tid + kStage * kSendBlock; c < chunks; c += kSendBlock)
        *reinterpret_cast<u32x4*>(msg + 4 + 16 * c) = src[c];
      __syncthreads();
      if (i + 1 < n) load_row<kStage>(v, src_row(i + 1), chunks);
      const int e = __builtin_amdgcn_readlane(e_l, i);
      if (t >= 0 && t < P.max_tokens)
        copy_message<true>(P.stage + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)t) * mc, msg, mc);
    }

    // release: this wave's stores are complete, then every wave's; wave 0
    // adds per distinct expert the number of rows staged for it to the
    // word's high half (little-endian: byte offset 4)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid < kWave) {
      const int e = lane < n && t_l >= 0 && t_l < P.max_tokens ? e_l : -1;
      int group = 0;
      for_each_distinct(e, [&](int val, uint64_t same) {
        if (e == val && (same & lanes_below()) == 0) group = __popcll(same);
      });
      if (group > 0)
        __hip_atomic_fetch_add(reinterpret_cast<unsigned int*>(P.sig + e) + 1, (unsigned int)group,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The same staging straight from registers, for batches below
// kSendLineBytes (their rows stay in L2 and MALL): every thread keeps the
// 16-byte chunks of the output row it loaded and stores them at staging
// byte 4 + 16c, dword-aligned stores at the row's own 4-byte phase, so no
// LDS copy and no barrier come between a row's loads and its stores; the
// next row's loads are issued before the current row's stores.
__device__ __forceinline__ void stage_rows_direct(const SendParams& P, uint32_t* pre, uint32_t r0,
                                                  uint32_t r1) {
  constexpr int kStage = 4;
  constexpr int kRound = kStage * kSendBlock;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int E = P.num_experts;
  const int chunks = P.hidden / 8;
  const uint32_t mc = P.comb_bytes;
  const u32x4* y = reinterpret_cast<const u32x4*>(P.y);

  for (uint32_t b0 = r0; b0 < r1; b0 += kWave) {
    const int n = r1 - b0 < (uint32_t)kWave ? (int)(r1 - b0) : kWave;
    // this lane's row of the batch: expert, slot and header
    const uint32_t r = b0 + (uint32_t)(lane < n ? lane : n - 1);
    const int e_l = expert_of_row(pre, E, r);
    const int j_l = (int)(r - pre[e_l]);
    const uint64_t src_l = (uint64_t)e_l * (uint64_t)P.max_tokens + (uint64_t)j_l;
    const int t_l = *reinterpret_cast<const int32_t*>(P.recv + src_l * P.msg_bytes);

    auto src_row = [&](int i) {
      const int e = __builtin_amdgcn_readlane(e_l, i);
      const int j = __builtin_amdgcn_readlane(j_l, i);
      return y + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)j) * (uint64_t)chunks;
    };
    u32x4 v[kStage];
    load_row<kStage>(v, src_row(0), chunks);
    for (int i = 0; i < n; ++i) {
      u32x4 nx[kStage];
      if (i + 1 < n) load_row<kStage>(nx, src_row(i + 1), chunks);
      const int t = __builtin_amdgcn_readlane(t_l, i);
      const int e = __builtin_amdgcn_readlane(e_l, i);
      if (t >= 0 && t < P.max_tokens) {
        const BufRsrc rsrc = message_rsrc(
            P.stage + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)t) * mc, mc);
        if (tid == 0) store_b32((uint32_t)t, rsrc, 0);
        put_chunks<kStage, kSendBlock>(rsrc, v, 0, 0, chunks);
        for (int cb = kRound; cb < chunks; cb += kRound) {  // rows wider than one round
          u32x4 w[kStage];
          load_row<kStage>(w, src_row(i), chunks, cb);
          put_chunks<kStage, kSendBlock>(rsrc, w, cb, 0, chunks);
        }
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u) v[u] = nx[u];
    }

    // release, as stage_rows
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid < kWave) {
      const int e = lane < n && t_l >= 0 && t_l < P.max_tokens ? e_l : -1;
      int group = 0;
      for_each_distinct(e, [&](int val, uint64_t same) {
        if (e == val && (same & lanes_below()) == 0) group = __popcll(same);
      });
      if (group > 0)
        __hip_atomic_fetch_add(reinterpret_cast<unsigned int*>(P.sig + e) + 1, (unsigned int)group,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void __launch_bounds__(kSendBlock) combine_send_kernel(const SendParams P) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  __shared__ uint32_t wave_sum[kSendBlock / kWave];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += blockDim.x) P.sig_other[e] = 0;

  // No acquire fence: the counts, headers and expert rows come from kernels
  // ordered before this one (stream order or events), and a kernel boundary
  // already makes their writes visible. An in-kernel acquire at device scope
  // invalidates the XCD's L2; one per workgroup costs ~27 us per launch.
  uint32_t* pre = reinterpret_cast<uint32_t*>(lds_raw);
  const uint32_t rows = load_count_prefix(P.sig, P.num_experts, P.max_tokens, pre, wave_sum);

  const uint32_t r0 = (uint32_t)((uint64_t)rows * blockIdx.x / gridDim.x);
  const uint32_t r1 = (uint32_t)((uint64_t)rows * (blockIdx.x + 1) / gridDim.x);
  if (r0 >= r1) return;
  uint8_t* lds_msg = lds_raw + count_prefix_bytes(P.num_experts) + kMsgLdsOffset;
  const uint32_t msg_stride = ((uint32_t)kMsgLdsOffset + P.comb_bytes + 15u) & ~15u;
  if ((uint64_t)rows * P.comb_bytes >= kSendLineBytes)
    stage_rows(P, pre, lds_msg, msg_stride, P.nbuf, r0, r1);
  else
    stage_rows_direct(P, pre, r0, r1);
}

hipError_t launch_combine_send(const SendParams& p, int blocks, hipStream_t stream) {
  const uint32_t msg_stride = ((uint32_t)kMsgLdsOffset + p.comb_bytes + 15u) & ~15u;
  const size_t lds = count_prefix_bytes(p.num_experts) + (size_t)p.nbuf * msg_stride;
  combine_send_kernel<<<blocks, kSendBlock, lds, stream>>>(p);
  return hipGetLastError();
}

// The gather-fold of NT consecutive tokens t0.. over this thread's 8
// columns, once the flags are up. Lane k of the wavefront holds token i's
// pick k's expert (e_l[i], or -1 when masked) and weight (w_l[i]); every
// load is issued before any is used; a masked pick borrows a routed pick's
// row of its token (its expert-0 row when none is routed) so that the loads
// stay unconditional, with no branch between them, and its value is never
// used.
//
// The staged payload is read with device-coherent buffer loads (sc1): like
// the flag polls, they are served at device scope and never from a stale L2
// line, and they are issued only after the polls have returned the raised
// flags, whose rows were complete in memory before the flags were added.
// That takes the place of an acquire fence, which would invalidate the
// XCD's L2 once per wavefront and token (14 us of an 18 us launch at 128
// tokens). The descriptor of pick k covers its one staging row.
template <int NT, int MAXK, bool STREAM>
__device__ __forceinline__ void fold_tokens(const RecvParams& P, int t0, int c,
                                            const int (&e_l)[NT], const float (&w_l)[NT]) {
  constexpr int kPolicy = STREAM ? kCachePolicySc1 | kCachePolicyNt : kCachePolicySc1;
  bool routed[NT][MAXK];
  float w[NT][MAXK];
  u32x4 v[NT][MAXK];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    uint64_t row[MAXK];
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const int e = __builtin_amdgcn_readlane(e_l[i], k < P.topk ? k : 0);
      routed[i][k] = k < P.topk && e >= 0;
      row[k] = (uint64_t)(routed[i][k] ? e : 0) * (uint64_t)P.max_tokens + (uint64_t)(t0 + i);
      w[i][k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l[i]),
                                                         k < P.topk ? k : 0));
    }
    uint64_t fallback = (uint64_t)(t0 + i);
#pragma unroll
    for (int k = MAXK - 1; k >= 0; --k) fallback = routed[i][k] ? row[k] : fallback;
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const BufRsrc rsrc = message_rsrc(
          const_cast<uint8_t*>(P.stage) + (routed[i][k] ? row[k] : fallback) * P.comb_bytes,
          P.comb_bytes);
      v[i][k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, 4 + 16 * c, 0, kPolicy);
    }
  }
  const int chunks = P.hidden / 8;
  fold_store<NT, MAXK>(v, routed, w, [&](int i) {
    return reinterpret_cast<gf32x4*>(P.out) + (uint64_t)(t0 + i) * (uint64_t)(chunks * 2) +
           2 * (uint64_t)c;
  });
}

template <int MAXK, bool STREAM>
__global__ void __launch_bounds__(kCombineMaxBlock) combine_recv_kernel(const RecvParams P) {
  const int tid = threadIdx.x;
  const int E = P.num_experts;
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += blockDim.x) P.sig_other[e] = 0;

  // 1. bounded wait for the flags. Workgroup 0 polls every expert's flag
  //    (high half == low half; an expert that received nothing is up) and
  //    posts the outcome in the status word (with the waited bit when its
  //    first look found a flag down); the other workgroups poll that one
  //    word. Per-token polling by every workgroup put K flag lines per
  //    workgroup and round onto the memory channel holding the signal words,
  //    which slowed the expert side it was waiting for (decode size: expert
  //    start to folded output 24 us overlapped against 15 us queued after).
  __shared__ int32_t posted;
  if (blockIdx.x == 0) {
    bool up = false;
    int32_t waited = 0;
    for (int spins = 1;; ++spins) {
      bool pending = false;
      for (int e = tid; e < E; e += blockDim.x) {
        const uint64_t s = __hip_atomic_load(P.sig + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pending = pending || (uint32_t)(s >> 32) != (uint32_t)s;
      }
      if (!__syncthreads_or(pending)) {
        up = true;
        waited = spins > 1 ? kStatusWaited : 0;
        break;
      }
      if (spins >= P.max_spins) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0)
      __hip_atomic_fetch_or(P.status, up ? kStatusReady | waited : kRefusalFlagWait,
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!up) return;
  } else {
    // A follower looks at the flags once itself (queued after the expert
    // side they are up, and it need not wait for workgroup 0's post); if
    // some are down it polls the status word, at most twice as many rounds
    // as workgroup 0 polls.
    bool pending = false;
    for (int e = tid; e < E; e += blockDim.x) {
      const uint64_t s = __hip_atomic_load(P.sig + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pending = pending || (uint32_t)(s >> 32) != (uint32_t)s;
    }
    const int limit = !__syncthreads_or(pending) ? 0
                      : P.max_spins > (1 << 29) ? (1 << 30) : 2 * P.max_spins + 64;
    for (int spins = 1; limit > 0; ++spins) {
      if (tid == 0) {
        int32_t v = __hip_atomic_load(P.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v == 0 && spins >= limit) {
          __hip_atomic_fetch_or(P.status, kRefusalFlagWait, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
          v = kRefusalFlagWait;
        }
        posted = v;
      }
      __syncthreads();
      const int32_t v = posted;
      __syncthreads();  // read everywhere before thread 0 writes it again
      if (v & kRefusalFlagWait) return;
      if (v & kStatusReady) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }

  // 2. fold. Work items are (tile of tokens, run of columns) pairs; a
  //    bounded grid loops over them, so that a token side started before
  //    the expert side leaves the GPU room to run the expert side.
  const int chunks = P.hidden / 8;
  const int lane = tid & (kWave - 1);
  const int tiles = (P.num_tokens + P.tile - 1) / P.tile;
  const int items = tiles * P.slices;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int tile = item / P.slices;
    const int sl = item - tile * P.slices;
    const int t0 = tile * P.tile;
    const int t1 = t0 + P.tile < P.num_tokens ? t0 + P.tile : P.num_tokens;
    const int c = sl * (int)blockDim.x + tid;
    // A wavefront wholly past the row has nothing to do. In the others every
    // lane loads its pick, also lanes past the row: fold_tokens reads picks
    // from lanes 0..topk-1 with readlane, which ignores the execution mask,
    // so those lanes must hold the tokens' values.
    if (sl * (int)blockDim.x + (tid & ~(kWave - 1)) >= chunks) continue;
    auto pick = [&](int t, int& e_l, float& w_l) {
      e_l = -1;
      w_l = 0.0f;
      if (lane < P.topk) {
        const int e = P.idx[(uint64_t)t * P.topk + lane];
        e_l = e >= 0 && e < E ? e : -1;
        w_l = P.w[(uint64_t)t * P.topk + lane];
      }
    };
    if (MAXK <= 8 && t1 - t0 == 2) {  // both tokens' loads in flight, as the fused combine
      int e_l[2];
      float w_l[2];
      pick(t0, e_l[0], w_l[0]);
      pick(t0 + 1, e_l[1], w_l[1]);
      if (c < chunks) fold_tokens<2, MAXK, STREAM>(P, t0, c, e_l, w_l);
    } else {
      for (int t = t0; t < t1; ++t) {
        int e_l[1];
        float w_l[1];
        pick(t, e_l[0], w_l[0]);
        if (c < chunks) fold_tokens<1, MAXK, STREAM>(P, t, c, e_l, w_l);
      }
    }
  }
}

template <bool STREAM>
static void launch_recv_k(const RecvParams& p, int blocks, hipStream_t stream) {
  if (p.topk <= 2)
    combine_recv_kernel<2, STREAM><<<blocks, p.block, 0, stream>>>(p);
  else if (p.topk <= 4)
    combine_recv_kernel<4, STREAM><<<blocks, p.block, 0, stream>>>(p);
  else if (p.topk <= 8)
    combine_recv_kernel<8, STREAM><<<blocks, p.block, 0, stream>>>(p);
  else
    combine_recv_kernel<16, STREAM><<<blocks, p.block, 0, stream>>>(p);
}

hipError_t launch_combine_recv(const RecvParams& p, hipStream_t stream) {
  const int tiles = p.num_tokens > 0 ? (p.num_tokens + p.tile - 1) / p.tile : 1;
  const int blocks = tiles * p.slices < kRecvBlocks ? tiles * p.slices : kRecvBlocks;
  if (p.stream_rows)
    launch_recv_k<true>(p, blocks, stream);
  else
    launch_recv_k<false>(p, blocks, stream);
  return hipGetLastError();
}

}  // namespace llmoe
