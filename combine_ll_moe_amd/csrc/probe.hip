// Measurement probes (declared in include/ll_moe_diag.h): plain kernels that
// move the bytes of the path's kernels without the rest of their work, so
// that the path can be placed against what the part itself does.
//
//  - stream: a contiguous write, read or copy of a large buffer, 16-byte
//    accesses, four in flight per thread: the practical HBM ceilings; and a
//    fold that reads four bytes for every byte it writes (the combine's
//    proportions at top-k 8), sixteen loads in flight per thread.
//  - store_rows: the dispatch's stores alone. Every listed destination row
//    receives row_bytes bytes of a pattern through one of the dispatch's
//    own store routines: from an LDS buffer by workgroup (copy_message) or
//    by wavefront (copy_row_wave), destination-aligned 16-byte buffer
//    stores, optionally whole-line dealing; or straight from registers
//    (put_chunks, as the dispatch writes batches below 64 MiB). No loads of
//    x, no routing and no count publish.
//  - gather_rows: the combine's gather alone. Each token folds the listed
//    expert-output rows through the combine's own gather_tile, in the
//    combine's launch shape, with no routing prologue.
// None of them is part of the step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ll_moe.h"
#include "ll_moe_diag.h"
#include "gather.h"
#include "kernels.h"
#include "layout.h"
#include "message.h"

namespace llmoe {
namespace {

constexpr int kProbeBlock = 256;
constexpr int kStreamUnroll = 4;
constexpr int kFoldSources = 4;  // source regions of the fold: 4 bytes read per byte written
constexpr int kMaxRowsPerBlock = kProbeBlock;

// Workgroup b streams tiles b, b + grid, ... of kProbeBlock * kStreamUnroll
// 16-byte chunks (16 KiB), each tile contiguous: every wavefront store or
// load covers 1 KiB, and a workgroup's four in flight cover 16 KiB (the
// fold: the same tile of each of its four source regions, 64 KiB).
template <int MODE, bool NT>
__global__ void __launch_bounds__(kProbeBlock)
    stream_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, uint64_t n,
                  uint32_t pattern) {
  constexpr uint64_t kTile = (uint64_t)kProbeBlock * kStreamUnroll;
  uint32_t acc = 0;
  for (uint64_t t0 = (uint64_t)blockIdx.x * kTile; t0 < n; t0 += (uint64_t)gridDim.x * kTile) {
    if constexpr (MODE == LL_MOE_PROBE_WRITE) {
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint64_t j = t0 + (uint64_t)u * kProbeBlock + threadIdx.x;
        const u32x4 v = {pattern, pattern ^ 1u, pattern ^ 2u, (uint32_t)j};
        if (j < n) {
          if (NT)
            __builtin_nontemporal_store(v, dst + j);
          else
            dst[j] = v;
        }
      }
    } else if constexpr (MODE == LL_MOE_PROBE_FOLD4) {
      // dst[j] = src[j] + src[n + j] + src[2n + j] + src[3n + j], lane-wise
      u32x4 v[kStreamUnroll][kFoldSources];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint64_t j = t0 + (uint64_t)u * kProbeBlock + threadIdx.x;
        const uint64_t jj = j < n ? j : n - 1;
#pragma unroll
        for (int k = 0; k < kFoldSources; ++k)
          v[u][k] = NT ? __builtin_nontemporal_load(src + k * n + jj) : src[k * n + jj];
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint64_t j = t0 + (uint64_t)u * kProbeBlock + threadIdx.x;
        const u32x4 f = v[u][0] + v[u][1] + v[u][2] + v[u][3];
        if (j < n) {
          if (NT)
            __builtin_nontemporal_store(f, dst + j);
          else
            dst[j] = f;
        }
      }
    } else {
      u32x4 v[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint64_t j = t0 + (uint64_t)u * kProbeBlock + threadIdx.x;
        const uint64_t jj = j < n ? j : n - 1;
        v[u] = NT ? __builtin_nontemporal_load(src + jj) : src[jj];
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const uint64_t j = t0 + (uint64_t)u * kProbeBlock + threadIdx.x;
        if constexpr (MODE == LL_MOE_PROBE_READ) {
          acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else if (j < n) {
          if (NT)
            __builtin_nontemporal_store(v[u], dst + j);
          else
            dst[j] = v[u];
        }
      }
    }
  }
  // a read must have a consumer: one word, written only when the fold
  // happens to equal the pattern
  if constexpr (MODE == LL_MOE_PROBE_READ)
    if (acc == pattern) dst[0].x = acc;
}

template <int MODE>
hipError_t launch_stream_mode(bool nt, u32x4* dst, const u32x4* src, uint64_t n, int blocks,
                              hipStream_t stream) {
  if (nt)
    stream_kernel<MODE, true><<<blocks, kProbeBlock, 0, stream>>>(dst, src, n, 0x5A5A5A5Au);
  else
    stream_kernel<MODE, false><<<blocks, kProbeBlock, 0, stream>>>(dst, src, n, 0x5A5A5A5Au);
  return hipGetLastError();
}

// Workgroup b writes rows [b * per, (b + 1) * per) of the list. Its LDS
// holds the row offsets, then one message buffer at the dispatch's LDS
// placement filled with a pattern.
template <bool LINE, int POLICY, bool WAVE_ROWS>
__global__ void __launch_bounds__(kProbeBlock)
    store_rows_kernel(uint8_t* base, const int64_t* __restrict__ off, int nrows,
                      uint32_t row_bytes, int per, uint32_t offs_bytes) {
  extern __shared__ __align__(16) uint8_t lds[];
  int64_t* offs = reinterpret_cast<int64_t*>(lds);
  uint8_t* msg = lds + offs_bytes + kMsgLdsOffset;
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * per;
  const int r1 = r0 + per < nrows ? r0 + per : nrows;
  if (tid < r1 - r0) offs[tid] = off[r0 + tid];
  for (uint32_t b = 4u * tid; b < row_bytes; b += 4u * blockDim.x)
    *reinterpret_cast<uint32_t*>(msg + b) = 0xC3C30000u ^ b;
  __syncthreads();
  if constexpr (WAVE_ROWS) {
    // the dispatch's wavefront rows: wavefront w writes rows w, w + 4, ...
    constexpr int kWaves = kProbeBlock / 64;
    for (int r = r0 + tid / 64; r < r1; r += kWaves)
      copy_row_wave<LINE, POLICY>(base + offs[r - r0], msg, row_bytes);
  } else {
    for (int r = r0; r < r1; ++r) copy_message<LINE, POLICY>(base + offs[r - r0], msg, row_bytes);
  }
}

// Rows straight from registers: workgroup b writes rows [b * per, (b + 1)
// * per) of the list, each by all its threads, the pattern computed in
// registers round by round (rows of a 4-byte header and whole 16-byte
// chunks).
template <int POLICY>
__global__ void __launch_bounds__(kProbeBlock)
    store_rows_direct_kernel(uint8_t* base, const int64_t* __restrict__ off, int nrows,
                             uint32_t row_bytes, int per) {
  constexpr int kStage = 4;
  constexpr int kRound = kStage * kProbeBlock;
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * per;
  const int r1 = r0 + per < nrows ? r0 + per : nrows;
  const int chunks = (int)((row_bytes - 4u) / 16u);
  for (int cb = 0; cb < chunks; cb += kRound) {  // uniform
    u32x4 v[kStage];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const uint32_t b = 4u + 16u * (uint32_t)(cb + tid + s * kProbeBlock);
      v[s] = u32x4{0xC3C30000u ^ b, 0xC3C30000u ^ (b + 4u), 0xC3C30000u ^ (b + 8u),
                   0xC3C30000u ^ (b + 12u)};
    }
    for (int r = r0; r < r1; ++r) {
      const BufRsrc rs = message_rsrc(base + off[r], row_bytes);
      if (cb == 0 && tid == 0) store_b32<POLICY>(0xC3C30000u, rs, 0);
      put_chunks<kStage, kProbeBlock, POLICY>(rs, v, cb, 0, chunks);
    }
  }
}

hipError_t launch_store_rows_direct(int policy, uint8_t* base, const int64_t* off, int nrows,
                                    uint32_t row_bytes, int per, hipStream_t stream) {
  const int blocks = (nrows + per - 1) / per;
#define LLMOE_STORE_DIRECT(POL) \
  store_rows_direct_kernel<POL><<<blocks, kProbeBlock, 0, stream>>>(base, off, nrows, row_bytes, per)
  switch (policy) {
    case LL_MOE_PROBE_SC1:
      LLMOE_STORE_DIRECT(kCachePolicySc1);
      break;
    case LL_MOE_PROBE_WRITE_BACK:
      LLMOE_STORE_DIRECT(0);
      break;
    case LL_MOE_PROBE_NT:
      LLMOE_STORE_DIRECT(kCachePolicyNt);
      break;
    default:
      LLMOE_STORE_DIRECT(kCachePolicySc1 | kCachePolicyNt);
      break;
  }
#undef LLMOE_STORE_DIRECT
  return hipGetLastError();
}

template <bool LINE, bool WAVE_ROWS>
hipError_t launch_store_rows_policy(int policy, uint8_t* base, const int64_t* off, int nrows,
                                    uint32_t row_bytes, int per, hipStream_t stream) {
  const uint32_t offs_bytes = ((uint32_t)per * 8u + 15u) & ~15u;
  const size_t lds = offs_bytes + ((kMsgLdsOffset + row_bytes + 15u) & ~15u);
  const int blocks = (nrows + per - 1) / per;
#define LLMOE_STORE_ROWS(POL)                                                                 \
  store_rows_kernel<LINE, POL, WAVE_ROWS>                                                     \
      <<<blocks, kProbeBlock, lds, stream>>>(base, off, nrows, row_bytes, per, offs_bytes)
  switch (policy) {
    case LL_MOE_PROBE_SC1:
      LLMOE_STORE_ROWS(kCachePolicySc1);
      break;
    case LL_MOE_PROBE_WRITE_BACK:
      LLMOE_STORE_ROWS(0);
      break;
    case LL_MOE_PROBE_NT:
      LLMOE_STORE_ROWS(kCachePolicyNt);
      break;
    default:
      LLMOE_STORE_ROWS(kCachePolicySc1 | kCachePolicyNt);
      break;
  }
#undef LLMOE_STORE_ROWS
  return hipGetLastError();
}

// The combine's work items, rows handed in: workgroup -> (tile of tokens,
// run of columns), the tile's picks gathered and folded by gather_tile. A row outside
// [0, y_rows) (a masked pick is -1) takes no part.
template <int MAXK, bool STREAM>
__global__ void __launch_bounds__(kCombineMaxBlock)
    gather_rows_kernel(const g32x4* __restrict__ y, int64_t y_rows, const int32_t* __restrict__ rows,
                       const float* __restrict__ wt, gf32x4* __restrict__ out, int num_tokens,
                       int topk, int chunks, int tile, int slices) {
  const int tl = blockIdx.x / slices;
  const int sl = blockIdx.x - tl * slices;
  const int t0 = tl * tile;
  const int c = sl * (int)blockDim.x + threadIdx.x;
  if (t0 >= num_tokens || c >= chunks) return;
  const int t1 = t0 + tile < num_tokens ? t0 + tile : num_tokens;
  auto tok = [&](int i, uint64_t (&row)[MAXK], bool (&routed)[MAXK], float (&w)[MAXK]) {
    const int t = t0 + i;
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const int kk = k < topk ? k : 0;
      const int r = rows[(uint64_t)t * topk + kk];
      routed[k] = k < topk && r >= 0 && (int64_t)r < y_rows;
      row[k] = routed[k] ? (uint64_t)r : 0;
      w[k] = wt[(uint64_t)t * topk + kk];
    }
  };
  auto dst = [&](int i) {
    return out + (uint64_t)(t0 + i) * (uint64_t)(chunks * 2) + 2 * (uint64_t)c;
  };
  gather_tile<MAXK, STREAM>(y, t1 - t0, c, chunks, tok, dst);
}

template <bool STREAM>
void launch_gather_rows_k(int blocks, const g32x4* y, int64_t y_rows, const int32_t* rows,
                          const float* wt, gf32x4* out, int num_tokens, int topk, int chunks,
                          int tile, int slices, int block, hipStream_t stream) {
#define LLMOE_GATHER(K)                                                                      \
  gather_rows_kernel<K, STREAM><<<blocks, block, 0, stream>>>(                               \
      y, y_rows, rows, wt, out, num_tokens, topk, chunks, tile, slices)
  if (topk <= 2)
    LLMOE_GATHER(2);
  else if (topk <= 4)
    LLMOE_GATHER(4);
  else if (topk <= 8)
    LLMOE_GATHER(8);
  else
    LLMOE_GATHER(16);
#undef LLMOE_GATHER
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
int from_hip(hipError_t e) { return e == hipSuccess ? LL_MOE_SUCCESS : LL_MOE_HIP_ERROR; }

}  // namespace
}  // namespace llmoe

using namespace llmoe;

extern "C" int ll_moe_diag_stream(int mode, int non_temporal, void* dst, const void* src,
                                  size_t bytes, int blocks, hipStream_t stream) {
  if (mode != LL_MOE_PROBE_WRITE && mode != LL_MOE_PROBE_READ && mode != LL_MOE_PROBE_COPY &&
      mode != LL_MOE_PROBE_FOLD4)
    return LL_MOE_INVALID_ARGUMENT;
  if (blocks < 1 || bytes % 16 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (bytes == 0) return LL_MOE_SUCCESS;
  if (!dst || !aligned(dst, 16)) return LL_MOE_INVALID_ARGUMENT;
  if (mode != LL_MOE_PROBE_WRITE && (!src || !aligned(src, 16))) return LL_MOE_INVALID_ARGUMENT;
  const uint64_t n = bytes / 16;
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  hipError_t e;
  if (mode == LL_MOE_PROBE_WRITE)
    e = launch_stream_mode<LL_MOE_PROBE_WRITE>(non_temporal != 0, d, s, n, blocks, stream);
  else if (mode == LL_MOE_PROBE_READ)
    e = launch_stream_mode<LL_MOE_PROBE_READ>(non_temporal != 0, d, s, n, blocks, stream);
  else if (mode == LL_MOE_PROBE_COPY)
    e = launch_stream_mode<LL_MOE_PROBE_COPY>(non_temporal != 0, d, s, n, blocks, stream);
  else
    e = launch_stream_mode<LL_MOE_PROBE_FOLD4>(non_temporal != 0, d, s, n, blocks, stream);
  return from_hip(e);
}

extern "C" int ll_moe_diag_store_rows(void* base, const int64_t* row_offsets, int nrows,
                                      int row_bytes, int rows_per_block, int line, int rows,
                                      int policy, hipStream_t stream) {
  if (nrows < 0 || row_bytes < 4 || row_bytes % 4 != 0 ||
      (uint64_t)row_bytes > kMaxMessageBytes)
    return LL_MOE_INVALID_ARGUMENT;
  if (rows_per_block < 1 || rows_per_block > kMaxRowsPerBlock) return LL_MOE_INVALID_ARGUMENT;
  if (policy < LL_MOE_PROBE_SC1 || policy > LL_MOE_PROBE_SC1_NT) return LL_MOE_INVALID_ARGUMENT;
  if (rows < LL_MOE_PROBE_ROWS_GROUP || rows > LL_MOE_PROBE_ROWS_DIRECT)
    return LL_MOE_INVALID_ARGUMENT;
  if (rows == LL_MOE_PROBE_ROWS_DIRECT && (row_bytes - 4) % 16 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (nrows == 0) return LL_MOE_SUCCESS;
  if (!base || !row_offsets || !aligned(base, 16) || !aligned(row_offsets, 8))
    return LL_MOE_INVALID_ARGUMENT;
  uint8_t* b = static_cast<uint8_t*>(base);
  const uint32_t rb = (uint32_t)row_bytes;
  const bool wave = rows == LL_MOE_PROBE_ROWS_WAVE;
  hipError_t e;
  if (rows == LL_MOE_PROBE_ROWS_DIRECT)
    e = launch_store_rows_direct(policy, b, row_offsets, nrows, rb, rows_per_block, stream);
  else if (line)
    e = wave ? launch_store_rows_policy<true, true>(policy, b, row_offsets, nrows, rb,
                                                    rows_per_block, stream)
             : launch_store_rows_policy<true, false>(policy, b, row_offsets, nrows, rb,
                                                     rows_per_block, stream);
  else
    e = wave ? launch_store_rows_policy<false, true>(policy, b, row_offsets, nrows, rb,
                                                     rows_per_block, stream)
             : launch_store_rows_policy<false, false>(policy, b, row_offsets, nrows, rb,
                                                      rows_per_block, stream);
  return from_hip(e);
}

extern "C" int ll_moe_diag_gather_rows(const void* y, long long y_rows, int hidden,
                                       const int32_t* rows, const float* weights, int num_tokens,
                                       int topk, float* out, hipStream_t stream) {
  if (num_tokens < 0 || hidden < 8 || hidden % 8 != 0 || topk < 1 || topk > LL_MOE_MAX_TOPK ||
      y_rows < 1)  // a token with no pick in range still loads row 0
    return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens == 0) return LL_MOE_SUCCESS;
  if (!y || !rows || !weights || !out || !aligned(y, 16) || !aligned(out, 16) ||
      !aligned(rows, 4) || !aligned(weights, 4))
    return LL_MOE_INVALID_ARGUMENT;
  if ((int64_t)num_tokens * topk > INT32_MAX) return LL_MOE_INVALID_ARGUMENT;
  const int chunks = hidden / 8;
  const bool stream_rows = (uint64_t)num_tokens * topk * hidden * 2 >= kStreamRowsBytes;
  const CombineShape shape = combine_shape(num_tokens, hidden, topk, stream_rows);
  const int blocks = ((num_tokens + shape.tile - 1) / shape.tile) * shape.slices;
  const g32x4* yy = static_cast<const g32x4*>(y);
  gf32x4* o = reinterpret_cast<gf32x4*>(out);
  if (stream_rows)
    launch_gather_rows_k<true>(blocks, yy, y_rows, rows, weights, o, num_tokens, topk, chunks,
                               shape.tile, shape.slices, shape.block, stream);
  else
    launch_gather_rows_k<false>(blocks, yy, y_rows, rows, weights, o, num_tokens, topk, chunks,
                                shape.tile, shape.slices, shape.block, stream);
  return from_hip(hipGetLastError());
}
