// Dispatch: pack every token's top-k messages into per-expert receive slots.
//
// What is computed (rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, struct
// LLMoEBuffer and the LLMoEBufferLayout constructor): message(t) = int32 t
// followed by the payload; it goes to send row t and to receive row
// e * max_tokens + slot(t, k) for every routed pick; each expert's int64
// signal word is then raised by the number of messages it received, after
// the messages themselves (mscclpp.h, the put-then-signal contract above
// struct mscclppDevConn).
//
// Design on gfx950:
//  - One or more workgroups per token. A workgroup builds message(t) once
//    in LDS (bf16: a 16-byte-aligned copy of the row; fp8: quantized there),
//    computes the token's slots (route.h), then streams the message from LDS
//    to each of its destinations.
//  - Message rows are 4 + 2h bytes apart, so a destination starts at any
//    4-byte phase. Stores are aligned to the destination instead: 0-3 head
//    dwords, then whole 16-byte global_store_dwordx4 chunks, then 0-3 tail
//    dwords; the LDS side absorbs the phase (dword-granular LDS reads).
//  - The (message, chunk) pairs of a workgroup are dealt to its threads as
//    one flat sequence, so the last round of one message does not idle
//    threads while the next message waits.
//  - Messages are written with device-coherent (write-through) stores;
//    every wave waits for its own stores, then after a workgroup barrier
//    one lane per routed pick adds 1 to the expert's signal word with a
//    device-scope atomic. This is a release without an L2 write-back per
//    workgroup (which costs tens of microseconds over a launch). The other
//    set's signal words are zeroed by workgroup 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"
#include "route.h"

namespace llmoe {

constexpr int kDispatchBlock = 256;
// The message sits at this LDS byte offset, so that its payload (message
// byte 4) starts 16-byte aligned and the row of x lands with ds_write_b128.
constexpr int kMsgLdsOffset = 12;

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Message stores are buffer stores with the device-scope coherence bit
// (sc1): they write through the XCD's L2, so they are visible to every XCD
// once complete, and no L2 write-back is needed before the count is
// published. The buffer descriptor covers exactly one message, so a store
// can never leave it.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kCachePolicySc1 = 16;
constexpr int kBufferWord3 = 0x00020000;  // gfx9 raw-buffer format bits
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0)

__device__ __forceinline__ BufRsrc message_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ void store_b128(const u32x4_a4 v, BufRsrc r, uint32_t off) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, kCachePolicySc1);
}
__device__ __forceinline__ void store_b32(uint32_t v, BufRsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kCachePolicySc1);
}

// fp32 -> OCP e4m3 ("e4m3fn") code, round to nearest even, saturating to
// +-448; the infinities saturate and every NaN gives 0x7F. Integer form:
// normal codes round the fp32 mantissa at bit 20 and rebias the exponent
// (127 -> 7); below 2^-6 the code counts 2^-9 steps, taken with rint.
__device__ __forceinline__ uint32_t e4m3_code(float p) {
  const uint32_t u = __float_as_uint(p);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const float sub_steps = __uint_as_float(a < 0x3C800000u ? a : 0x3C800000u) * 512.0f;
  const uint32_t sub = (uint32_t)__builtin_rintf(sub_steps);
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t code = a < 0x3C800000u ? sub : (r >> 20) - (120u << 3);
  code = a >= 0x43E00000u ? 0x7Eu : code;  // |p| >= 448
  code |= sign;
  return a > 0x7F800000u ? 0x7Fu : code;   // NaN
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Eight elements (unit u) of the fp8 message; the 16 lanes of a block
// reduce amax together.
__device__ __forceinline__ void quantize_unit(uint8_t* msg, int hidden, int u, const u32x4 raw) {
  float f[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = __builtin_fabsf(f[j]);
    amax = a > amax ? a : amax;
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    const float o = __shfl_xor(amax, off, 16);
    amax = o > amax ? o : amax;
  }
  float inv = 0.0f, scale = 0.0f;
  if (amax > 0.0f) {
    inv = 448.0f / amax;
    scale = amax / 448.0f;
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) lo |= e4m3_code(f[j] * inv) << (8 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) hi |= e4m3_code(f[4 + j] * inv) << (8 * j);
  *reinterpret_cast<uint2*>(msg + 4 + 8 * u) = make_uint2(lo, hi);
  if ((u & 15) == 0) *reinterpret_cast<float*>(msg + 4 + hidden + 4 * (u >> 4)) = scale;
}

// fp8 message body: per 128-element block, amax over the block (NaN
// ignored), inv = 448 / amax and scale = amax / 448 (correctly rounded fp32
// divisions; both 0 when amax is 0), codes e4m3(x * inv), scales after the
// codes. Each thread takes 8 elements; a block is 16 consecutive lanes, and
// every lane of a 16-lane group is active together (hidden % 128 == 0 and
// the block size is a multiple of 64). r holds the first round's loads.
template <int NSTAGE>
__device__ __forceinline__ void stage_fp8(uint8_t* msg, const u32x4* __restrict__ xr, int hidden,
                                          const u32x4 (&r)[NSTAGE]) {
  const int units = hidden / 8;
  const int B = blockDim.x;
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) {
    const int u = threadIdx.x + s * B;
    if (u < units) quantize_unit(msg, hidden, u, r[s]);
  }
  for (int u0 = threadIdx.x + NSTAGE * B; u0 < units; u0 += NSTAGE * B) {
    u32x4 q[NSTAGE];
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s) {
      const int u = u0 + s * B;
      q[s] = xr[u < units ? u : units - 1];
    }
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s) {
      const int u = u0 + s * B;
      if (u < units) quantize_unit(msg, hidden, u, q[s]);
    }
  }
}

template <int DT, int MAXK>
__global__ void __launch_bounds__(kDispatchBlock) dispatch_kernel(const DispatchParams P) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  __shared__ RouteShared rs;
  __shared__ uint64_t s_dst[MAXK + 1];
  __shared__ int s_nmsg;

  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += blockDim.x) P.sig_other[e] = 0;

  const int t = blockIdx.x / P.groups;
  const int g = blockIdx.x - t * P.groups;
  if (t >= P.num_tokens) return;

  // 1. issue the loads of x[t] (first staging round) before the routing
  //    prologue so that both memory round trips overlap
  uint8_t* msg = lds_raw + kMsgLdsOffset;
  const u32x4* xr = reinterpret_cast<const u32x4*>(P.x) + (size_t)t * (P.hidden / 8);
  const int chunks = P.hidden / 8;
  constexpr int kStage = 4;
  u32x4 r[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int j = tid + u * (int)blockDim.x;
    r[u] = xr[j < chunks ? j : chunks - 1];  // unconditional: one wait for all
  }

  // 2. slots of token t
  route_token<MAXK>(P.idx, t, P.topk, P.num_experts, P.max_tokens, rs);

  // 3. message(t) in LDS: the preloaded round, then (rows longer than
  //    kStage * blockDim chunks only) the remaining rounds
  if (tid == 0) *reinterpret_cast<int32_t*>(msg) = t;
  if (DT == kBf16) {
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int j = tid + u * (int)blockDim.x;
      if (j < chunks) *reinterpret_cast<u32x4*>(msg + 4 + 16 * j) = r[u];
    }
    for (int j0 = tid + kStage * (int)blockDim.x; j0 < chunks; j0 += kStage * (int)blockDim.x) {
      u32x4 q[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int j = j0 + u * (int)blockDim.x;
        q[u] = xr[j < chunks ? j : chunks - 1];
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int j = j0 + u * (int)blockDim.x;
        if (j < chunks) *reinterpret_cast<u32x4*>(msg + 4 + 16 * j) = q[u];
      }
    }
  } else {
    stage_fp8<kStage>(msg, xr, P.hidden, r);
  }

  // 4. this workgroup's destinations: message m = g, g + groups, ... where
  //    m == topk is the send row (its barrier also publishes the LDS message)
  if (tid == 0) {
    int n = 0;
    for (int m = g; m <= P.topk; m += P.groups) {
      if (m == P.topk) {
        s_dst[n++] = (uint64_t)(P.send + (uint64_t)t * P.msg_bytes);
      } else if (rs.slot[m] >= 0) {
        const uint64_t row = (uint64_t)rs.expert[m] * (uint64_t)P.max_tokens + (uint64_t)rs.slot[m];
        s_dst[n++] = (uint64_t)(P.recv + row * P.msg_bytes);
      }
    }
    s_nmsg = n;
  }
  __syncthreads();

  // 5. stream LDS -> destinations with destination-aligned 16-byte stores.
  //    Per message: 0-3 head dwords and 0-3 tail dwords (one thread each),
  //    then the 16-byte body chunks, four per thread per round with the LDS
  //    reads of a round issued before its stores.
  const int nmsg = s_nmsg;
  const uint32_t md = P.msg_bytes;
  if (tid < nmsg) {
    void* d = reinterpret_cast<void*>(s_dst[tid]);
    const BufRsrc r = message_rsrc(d, md);
    const uint32_t head = (16u - ((uint32_t)(uintptr_t)d & 15u)) & 15u;
    const uint32_t body_end = head + ((md - head) & ~15u);
    for (uint32_t b = 0; b < head; b += 4) store_b32(*reinterpret_cast<const uint32_t*>(msg + b), r, b);
    for (uint32_t b = body_end; b < md; b += 4)
      store_b32(*reinterpret_cast<const uint32_t*>(msg + b), r, b);
  }
  constexpr int kCopy = 4;
  for (int mi = 0; mi < nmsg; ++mi) {
    void* d = reinterpret_cast<void*>(s_dst[mi]);
    const BufRsrc r = message_rsrc(d, md);
    const uint32_t head = (16u - ((uint32_t)(uintptr_t)d & 15u)) & 15u;
    const uint32_t nb = (md - head) >> 4;
    for (uint32_t i0 = tid; i0 < nb; i0 += kCopy * blockDim.x) {
      u32x4_a4 v[kCopy];
#pragma unroll
      for (int u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        v[u] = *reinterpret_cast<const u32x4_a4*>(msg + head + 16u * (i < nb ? i : nb - 1));
      }
#pragma unroll
      for (int u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        if (i < nb) store_b128(v[u], r, head + 16u * i);
      }
    }
  }
  // every wave waits until its own device-coherent stores are complete;
  // after the barrier, all of this workgroup's messages are visible at
  // device scope
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // 6. publish: one device-scope add per routed pick of this workgroup.
  //    The messages were written with device-coherent stores that have all
  //    completed (step 5), so the adds need no cache write-back of their
  //    own: a reader that loads the count with acquire semantics at device
  //    scope (which invalidates its L2 copy) sees the messages.
  if (tid < P.topk && (tid % P.groups) == g && rs.slot[tid] >= 0)
    __hip_atomic_fetch_add(P.sig + rs.expert[tid], 1ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT>
static hipError_t launch_dt(const DispatchParams& p, hipStream_t stream) {
  const int blocks = p.num_tokens > 0 ? p.num_tokens * p.groups : 1;
  const size_t lds = ((size_t)kMsgLdsOffset + p.msg_bytes + 15) & ~(size_t)15;
  if (p.topk <= 2)
    dispatch_kernel<DT, 2><<<blocks, kDispatchBlock, lds, stream>>>(p);
  else if (p.topk <= 4)
    dispatch_kernel<DT, 4><<<blocks, kDispatchBlock, lds, stream>>>(p);
  else if (p.topk <= 8)
    dispatch_kernel<DT, 8><<<blocks, kDispatchBlock, lds, stream>>>(p);
  else
    dispatch_kernel<DT, 16><<<blocks, kDispatchBlock, lds, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchParams& p, int dtype, hipStream_t stream) {
  return dtype == kBf16 ? launch_dt<kBf16>(p, stream) : launch_dt<kFp8>(p, stream);
}

// The fp8 encoder above, applied element-wise; lets a test compare it with
// an independent encoder on chosen fp32 inputs.
__global__ void e4m3_probe_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                  uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = (uint8_t)e4m3_code(in[i]);
}

hipError_t launch_e4m3_probe(const float* in, uint8_t* out, uint64_t n, hipStream_t stream) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  e4m3_probe_kernel<<<(unsigned)blocks, 256, 0, stream>>>(in, out, n);
  return hipGetLastError();
}

__global__ void clean_kernel(unsigned long long* sig, int n) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) sig[e] = 0;
}

hipError_t launch_clean(unsigned long long* sig, int num_experts, hipStream_t stream) {
  const int blocks = (num_experts + 255) / 256 < 64 ? (num_experts + 255) / 256 : 64;
  clean_kernel<<<blocks, 256, 0, stream>>>(sig, num_experts);
  return hipGetLastError();
}

}  // namespace llmoe
