// Message movement shared by the kernels that write messages for another
// workgroup or kernel to read (dispatch, two-phase combine expert side):
// register loads of a 16-byte-aligned row, and the stores of a message to
// its destination with device-coherent stores, from registers or from an
// LDS copy.
//
// Message stores are buffer stores with the device-scope coherence bit
// (sc1): they write through the XCD's L2, so they are visible to every XCD
// once complete, and no L2 write-back is needed before a signal word is
// raised. The buffer descriptor covers exactly one message, so a store can
// never leave it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace llmoe {

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t BufRsrc;

__device__ __forceinline__ BufRsrc message_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufferWord3);
}
template <int POLICY = kCachePolicySc1>
__device__ __forceinline__ void store_b128(const u32x4_a4 v, BufRsrc r, uint32_t off) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, POLICY);
}
template <int POLICY = kCachePolicySc1>
__device__ __forceinline__ void store_b64(uint2 v, BufRsrc r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)off, 0, POLICY);
}
template <int POLICY = kCachePolicySc1>
__device__ __forceinline__ void store_b32(uint32_t v, BufRsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, POLICY);
}

// NSTAGE * blockDim 16-byte chunks of a row into registers, from chunk
// `base` on (thread i takes chunks base + i + u * blockDim); unconditional
// loads with the index clamped into the row. STREAM: non-temporal loads,
// for rows read once.
template <int NSTAGE, bool STREAM = false>
__device__ __forceinline__ void load_row(u32x4 (&r)[NSTAGE], const u32x4* __restrict__ xr,
                                         int chunks, int base = 0) {
#pragma unroll
  for (int u = 0; u < NSTAGE; ++u) {
    const int j = base + (int)threadIdx.x + u * (int)blockDim.x;
    const u32x4* src = xr + (j < chunks ? j : chunks - 1);
    r[u] = STREAM ? __builtin_nontemporal_load(src) : *src;
  }
}

// Payload chunks of one round straight from registers into a message row:
// thread i holds chunks base + i + s * BLOCK (s < NS) in r[s] and stores
// those within [lo, hi) at row byte 4 + 16 * chunk, after the 4-byte
// header. The stores are 16-byte buffer stores at whatever 4-byte phase
// the row has (dword-aligned), of the given cache policy, confined to the
// message by the buffer descriptor; there is no LDS copy of the row.
template <int NS, int BLOCK, int POLICY = kCachePolicySc1>
__device__ __forceinline__ void put_chunks(BufRsrc rsrc, const u32x4 (&r)[NS], int base, int lo,
                                           int hi) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = base + tid + s * BLOCK;
    if (c >= lo && c < hi)
      store_b128<POLICY>(u32x4_a4{r[s].x, r[s].y, r[s].z, r[s].w}, rsrc, 4u + 16u * (uint32_t)c);
  }
}

// Part `part` of `parts` of one message, from LDS to its destination. The
// destination splits into 0-3 head dwords, whole 16-byte body chunks and
// 0-3 tail dwords; part p takes body chunks [nb * p / parts, nb * (p + 1) /
// parts), the first part also the head and the last the tail (one thread
// each). Body chunks go four per thread per round, with the round's LDS
// reads issued before its stores; the stores are destination-aligned,
// device-coherent, and confined to the message by the buffer descriptor.
//
// With LINE, chunks are dealt to lanes so that every 8 lanes write
// one whole 128-byte cache line: chunk k goes to virtual index k + sh, where
// sh is the body's 16-byte offset within its first line, and lanes of a
// round take consecutive virtual indices from a multiple of 8. A 1 KiB wave
// store then covers 8 whole lines instead of straddling 9; for write-through
// stores that go to HBM this is a quarter faster. (For data the caches
// absorb it costs a little, so the caller decides.)
// POLICY is the stores' cache policy: device-coherent write-through (sc1)
// for every message of the path; the measurement probes also time others.
template <bool LINE, int POLICY = kCachePolicySc1>
__device__ __forceinline__ void copy_message(void* d, const uint8_t* msg, uint32_t md,
                                             uint32_t part = 0, uint32_t parts = 1) {
  constexpr int kCopy = 4;
  const uint32_t tid = threadIdx.x;
  const BufRsrc rsrc = message_rsrc(d, md);
  const uint32_t head = (16u - ((uint32_t)(uintptr_t)d & 15u)) & 15u;
  const uint32_t nb = (md - head) >> 4;
  const uint32_t body_end = head + 16u * nb;
  const uint32_t c0 = nb * part / parts;
  const uint32_t c1 = nb * (part + 1) / parts;
  if (part == 0 && tid == 0)
    for (uint32_t b = 0; b < head; b += 4) store_b32<POLICY>(*reinterpret_cast<const uint32_t*>(msg + b), rsrc, b);
  if (part == parts - 1 && tid == 1)
    for (uint32_t b = body_end; b < md; b += 4) store_b32<POLICY>(*reinterpret_cast<const uint32_t*>(msg + b), rsrc, b);
  if constexpr (!LINE) {
    for (uint32_t i0 = c0 + tid; i0 < c1; i0 += kCopy * blockDim.x) {
      u32x4_a4 v[kCopy];
#pragma unroll
      for (int u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        v[u] = *reinterpret_cast<const u32x4_a4*>(msg + head + 16u * (i < c1 ? i : c1 - 1));
      }
#pragma unroll
      for (int u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * blockDim.x;
        if (i < c1) store_b128<POLICY>(v[u], rsrc, head + 16u * i);
      }
    }
    return;
  }
  if (c1 <= c0) return;
  // virtual indices [vlo, vend) hold chunks [c0, c1); a round starts at a
  // multiple of 8
  const uint32_t sh = (((uint32_t)(uintptr_t)d + head) & 127u) >> 4;
  const uint32_t vlo = c0 + sh;
  const uint32_t vend = c1 + sh;
  for (uint32_t v0 = (vlo & ~7u) + tid; v0 < vend; v0 += kCopy * blockDim.x) {
    u32x4_a4 v[kCopy];
#pragma unroll
    for (int u = 0; u < kCopy; ++u) {
      const uint32_t vi = v0 + u * blockDim.x;
      const uint32_t k = vi >= vlo && vi < vend ? vi - sh : c0;
      v[u] = *reinterpret_cast<const u32x4_a4*>(msg + head + 16u * k);
    }
#pragma unroll
    for (int u = 0; u < kCopy; ++u) {
      const uint32_t vi = v0 + u * blockDim.x;
      if (vi >= vlo && vi < vend) store_b128<POLICY>(v[u], rsrc, head + 16u * (vi - sh));
    }
  }
}

// Body chunks [a, b) of one message from LDS to its destination, written by
// one wavefront (all 64 lanes call it with the same arguments). The body
// starts `head` bytes into the destination (head = bytes to its first
// 16-byte boundary); chunk c is destination bytes [head + 16c, head + 16c +
// 16). Lane-strided, eight chunks per lane per round with the round's LDS
// reads issued before its stores; stores as in copy_message:
// destination-aligned, of the given cache policy, confined to the message
// by the buffer descriptor. LINE deals the chunks to lanes by whole 128-byte
// lines (every 8 lanes of a store cover one line).
template <bool LINE, int POLICY = kCachePolicySc1>
__device__ __forceinline__ void copy_body_wave(void* d, const uint8_t* msg, uint32_t md,
                                               uint32_t head, uint32_t a, uint32_t b) {
  constexpr uint32_t kCopy = 8;
  constexpr uint32_t kLanes = 64;
  const uint32_t lane = threadIdx.x & (kLanes - 1);
  const BufRsrc rsrc = message_rsrc(d, md);
  if constexpr (!LINE) {
    for (uint32_t i0 = a + lane; i0 < b; i0 += kCopy * kLanes) {
      u32x4_a4 v[kCopy];
#pragma unroll
      for (uint32_t u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * kLanes;
        v[u] = *reinterpret_cast<const u32x4_a4*>(msg + head + 16u * (i < b ? i : b - 1));
      }
#pragma unroll
      for (uint32_t u = 0; u < kCopy; ++u) {
        const uint32_t i = i0 + u * kLanes;
        if (i < b) store_b128<POLICY>(v[u], rsrc, head + 16u * i);
      }
    }
  } else {
    // virtual index vi = c + sh, sh = the body's 16-byte offset in its first
    // line; rounds start at multiples of 8
    const uint32_t sh = (((uint32_t)(uintptr_t)d + head) & 127u) >> 4;
    const uint32_t vlo = a + sh, vend = b + sh;
    for (uint32_t v0 = (vlo & ~7u) + lane; v0 < vend; v0 += kCopy * kLanes) {
      u32x4_a4 v[kCopy];
#pragma unroll
      for (uint32_t u = 0; u < kCopy; ++u) {
        const uint32_t vi = v0 + u * kLanes;
        const uint32_t k = vi >= vlo && vi < vend ? vi - sh : a;
        v[u] = *reinterpret_cast<const u32x4_a4*>(msg + head + 16u * k);
      }
#pragma unroll
      for (uint32_t u = 0; u < kCopy; ++u) {
        const uint32_t vi = v0 + u * kLanes;
        if (vi >= vlo && vi < vend) store_b128<POLICY>(v[u], rsrc, head + 16u * (vi - sh));
      }
    }
  }
}

// Bytes before a destination's first 16-byte boundary (at most md, whole
// dwords).
__device__ __forceinline__ uint32_t message_head(const void* d, uint32_t md) {
  const uint32_t head = (16u - ((uint32_t)(uintptr_t)d & 15u)) & 15u;
  return head < md ? head : md & ~3u;
}

// The 0-3 head dwords (bytes [0, head)) and 0-3 tail dwords (bytes
// [head + 16 * nb, md), nb = the whole body chunks) of one message, by lanes
// 0-2 of one wavefront.
template <int POLICY = kCachePolicySc1>
__device__ __forceinline__ void copy_edges_wave(void* d, const uint8_t* msg, uint32_t md,
                                                uint32_t head) {
  const uint32_t lane = threadIdx.x & 63u;
  const BufRsrc rsrc = message_rsrc(d, md);
  const uint32_t body_end = head + 16u * ((md - head) >> 4);
  if (4 * lane < head)
    store_b32<POLICY>(*reinterpret_cast<const uint32_t*>(msg + 4 * lane), rsrc, 4 * lane);
  if (body_end + 4 * lane < md)
    store_b32<POLICY>(*reinterpret_cast<const uint32_t*>(msg + body_end + 4 * lane), rsrc,
                      body_end + 4 * lane);
}

// One whole message from LDS to its destination, written by one wavefront
// (all 64 lanes call it with the same arguments): the head and tail dwords
// and every body chunk (copy_edges_wave, copy_body_wave).
template <bool LINE, int POLICY = kCachePolicySc1>
__device__ __forceinline__ void copy_row_wave(void* d, const uint8_t* msg, uint32_t md) {
  const uint32_t head = message_head(d, md);
  copy_edges_wave<POLICY>(d, msg, md, head);
  const uint32_t nb = (md - head) >> 4;
  if (nb > 0) copy_body_wave<LINE, POLICY>(d, msg, md, head, 0, nb);
}

}  // namespace llmoe
