// Expert side of the dispatch: wait until set q's messages are complete,
// then unpack them into the arrays an expert's matrix product reads.
//
// What is computed (rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, struct
// LLMoEBuffer's receive buffer and per-expert counts; mscclpp.h, the
// receiver reads only after the signal, above struct mscclppDevConn;
// memra-engine src/tp_ar.rs, a bounded device wait that leaves a refusal
// code): set q is complete once its counts (low halves of its signal words)
// add up to the number of messages the step routes; then for every expert e
// and j < count_e, receive row r = e * max_tokens + j gives payload row r
// (the message without its header: bf16 x bits, or the fp8 codes), scale
// row r (fp8: the h/128 scales), src[r] (the header) and counts[e].
//
// Design on gfx950: the launch may start while the dispatch is still
// running (on another stream), so its wait and its launch ramp hide behind
// the dispatch. Workgroup 0 polls the counts with relaxed device-scope
// loads and scans them in LDS until their sum reaches the expected number,
// at most max_spins times, and posts the outcome in a status word the
// caller zeroed (with a second bit when its first look found the set
// incomplete, so that a caller can tell that the call did overlap); every
// other workgroup looks at the counts once itself and, if they do not add
// up yet, polls that one word, then scans the (now final) counts. Each
// takes a contiguous run of the flattened (expert, slot) rows; each
// wavefront copies whole rows, so that a row's buffer descriptor is
// uniform and its payload can be read with device-coherent (sc1) loads.
// Those loads are served at device scope, like the polls, and issue after
// the polls have seen the full sum: they cannot return a stale L2 line, and
// no acquire fence (an L2 invalidate per workgroup) is needed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "expert.h"
#include "kernels.h"
#include "message.h"
#include "route.h"

namespace llmoe {

// KROUND: 16-byte loads in flight per lane before their stores (16 for
// the bandwidth-bound copies of 64 MiB or more: 1024 tokens of 7168
// columns 44.6 against 44.8 us with 8; 8 below, where 16 measured slower,
// 6.9 against 6.6 us at 128 tokens). STREAM_OUT: the payload rows go out
// with non-temporal stores, so that they do not evict from the MALL the
// receive rows still to be read (for 64 MiB or more: 1024 tokens of 7168
// columns unpacked in 39.0 against 45.1 us, and a dispatch followed by its
// unpack in 67.5 against 76.8). Below that size fp8 payloads stream too
// (128 tokens of 7168 columns: unpack 5.1 against 5.5 us, dispatch and
// unpack 13.2 against 13.5), bf16 ones do not (plain stores keep that pair
// shorter, 15.3 against 15.9 us, though the unpack alone is 6.0 against
// 6.6).
template <int KROUND, bool STREAM_OUT>
__global__ void __launch_bounds__(kSendBlock) dispatch_recv_kernel(const UnpackParams P) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  __shared__ uint32_t wave_sum[kSendBlock / kWave];
  const int tid = threadIdx.x;
  const int E = P.num_experts;
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += blockDim.x) P.sig_other[e] = 0;

  // 1. bounded wait. Workgroup 0 polls the counts, scanned in LDS, until
  //    their sum is the expected number of messages, at most max_spins
  //    times, and posts the outcome in the status word; the other
  //    workgroups poll only that word (one thread, then a barrier, so the
  //    whole workgroup takes one branch). Were every workgroup to poll all
  //    the counts, their loads would pile onto the few lines that the
  //    dispatch's count atomics also need, and slow the dispatch itself
  //    (measured: 8 -> 15 us at decode size).
  uint32_t* pre = reinterpret_cast<uint32_t*>(lds_raw);
  __shared__ int32_t posted;
  if (blockIdx.x == 0) {
    bool ready = false;
    int32_t waited = 0;
    for (int spins = 1;; ++spins) {
      // the sum is read after the scan's barrier: one value everywhere
      if (load_count_prefix(P.sig, E, P.max_tokens, pre, wave_sum) == (uint32_t)P.expected) {
        ready = true;
        waited = spins > 1 ? kStatusWaited : 0;
        break;
      }
      if (spins >= P.max_spins) break;
      __syncthreads();  // the sum is read everywhere before the next scan rewrites it
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0)
      __hip_atomic_fetch_or(P.status, ready ? kStatusReady | waited : kRefusalCountWait,
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!ready) return;
  } else if (load_count_prefix(P.sig, E, P.max_tokens, pre, wave_sum) != (uint32_t)P.expected) {
    // A follower looks at the counts once itself (queued after the dispatch
    // they are final, and it need not wait for workgroup 0's post); if they
    // do not add up yet it polls the status word, at most twice as many
    // rounds as workgroup 0 polls, its rounds being shorter.
    const int limit = P.max_spins > (1 << 29) ? (1 << 30) : 2 * P.max_spins + 64;
    for (int spins = 1;; ++spins) {
      if (tid == 0) {
        int32_t v = __hip_atomic_load(P.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v == 0 && spins >= limit) {
          __hip_atomic_fetch_or(P.status, kRefusalCountWait, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
          v = kRefusalCountWait;
        }
        posted = v;
      }
      __syncthreads();
      const int32_t v = posted;
      __syncthreads();  // read everywhere before thread 0 writes it again
      if (v & kRefusalCountWait) return;
      if (v & kStatusReady) break;
      __builtin_amdgcn_s_sleep(2);
    }
    // the counts are final now: workgroup 0 saw them add up before posting
    load_count_prefix(P.sig, E, P.max_tokens, pre, wave_sum);
  }
  const uint32_t rows = pre[kSendBlock * count_rounds(E)];
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += blockDim.x) P.counts[e] = (int32_t)(pre[e + 1] - pre[e]);

  // 2. this workgroup's rows, 64 at a time: lane l finds batch row l's
  //    expert and slot; wavefront w copies batch rows w, w + 4, ...
  const uint32_t r0 = (uint32_t)((uint64_t)rows * blockIdx.x / gridDim.x);
  const uint32_t r1 = (uint32_t)((uint64_t)rows * (blockIdx.x + 1) / gridDim.x);
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int waves = (int)blockDim.x / kWave;
  const uint32_t nch = P.row_bytes / 16;                 // 16-byte payload chunks per row
  const uint32_t nsc = P.fp8 ? (uint32_t)P.hidden / 128 : 0u;  // scales per row
  constexpr int kRound = KROUND;
  for (uint32_t b0 = r0; b0 < r1; b0 += kWave) {
    const int n = r1 - b0 < (uint32_t)kWave ? (int)(r1 - b0) : kWave;
    const uint32_t r = b0 + (uint32_t)(lane < n ? lane : n - 1);
    const int e_l = expert_of_row(pre, E, r);
    const int j_l = (int)(r - pre[e_l]);
    for (int i = wave; i < n; i += waves) {
      const int e = __builtin_amdgcn_readlane(e_l, i);
      const int j = __builtin_amdgcn_readlane(j_l, i);
      const uint64_t row = (uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)j;
      const BufRsrc msg = message_rsrc(const_cast<uint8_t*>(P.recv) + row * P.msg_bytes, P.msg_bytes);
      if (lane == 0) P.src[row] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(msg, 0, 0, kCachePolicySc1);
      u32x4* dst = reinterpret_cast<u32x4*>(P.payload + row * P.row_bytes);
      for (uint32_t c0 = lane; c0 < nch; c0 += kRound * kWave) {
        u32x4 v[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
          const uint32_t c = c0 + u * kWave;
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(msg, 4 + 16 * (c < nch ? c : nch - 1), 0,
                                                       kCachePolicySc1);
        }
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
          const uint32_t c = c0 + u * kWave;
          if (c < nch) {
            if constexpr (STREAM_OUT)
              __builtin_nontemporal_store(v[u], dst + c);
            else
              dst[c] = v[u];
          }
        }
      }
      for (uint32_t s = lane; s < nsc; s += kWave)
        P.scales[row * nsc + s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            msg, 4 + (int)P.row_bytes + 4 * (int)s, 0, kCachePolicySc1));
    }
  }
}

hipError_t launch_dispatch_recv(const UnpackParams& p, int blocks, hipStream_t stream) {
  if (p.wide)
    dispatch_recv_kernel<16, true>
        <<<blocks, kSendBlock, count_prefix_bytes(p.num_experts), stream>>>(p);
  else if (p.fp8)
    dispatch_recv_kernel<8, true>
        <<<blocks, kSendBlock, count_prefix_bytes(p.num_experts), stream>>>(p);
  else
    dispatch_recv_kernel<8, false>
        <<<blocks, kSendBlock, count_prefix_bytes(p.num_experts), stream>>>(p);
  return hipGetLastError();
}

}  // namespace llmoe
