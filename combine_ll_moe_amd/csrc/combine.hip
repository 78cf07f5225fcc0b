// Combine: gather the expert outputs back to their tokens as a top-k
// weighted sum.
//
// out[t, c] = fma chain over the routed picks k = 0..topk-1, in ascending k,
// of acc = fmaf(w[t, k], y[e * max_tokens + slot(t, k), c], acc), from
// +0.0f, in fp32. The operand order is fixed so that every call forms the
// same expression and returns the same bits (memra-engine src/tp_ar.rs,
// memra_tp_ar_1stage: both ranks' inputs are read in one global order).
// On one GPU the combine send/receive hand-off of the rocSHMEM example
// (struct LLMoEBuffer, combine buffers) becomes a direct gather from the
// expert outputs, as a one-shot reduction replaces push-then-fold.
//
// Design on gfx950: one workgroup per (token, run of columns). It computes
// the token's slots (route.h), then every thread issues its topk 16-byte
// loads of bf16 expert rows at once (all outstanding together), folds them
// with v_fma_f32 in k order, and writes 8 fp32 results as two 16-byte
// stores. Workgroup 0 zeroes the other set's signal words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"
#include "route.h"

namespace llmoe {

constexpr int kCombineBlock = 256;

template <int MAXK>
__global__ void __launch_bounds__(kCombineBlock) combine_kernel(const CombineParams P) {
  __shared__ RouteShared rs;
  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += blockDim.x) P.sig_other[e] = 0;

  const int t = blockIdx.x / P.slices;
  const int sl = blockIdx.x - t * P.slices;
  if (t >= P.num_tokens) return;

  route_token<MAXK>(P.idx, t, P.topk, P.num_experts, P.max_tokens, rs);

  const int chunks = P.hidden / 8;
  const int c = sl * blockDim.x + tid;
  if (c >= chunks) return;

  // Rows of the routed picks; a masked pick borrows the row of a routed
  // one so that every load is unconditional (the borrowed value is never
  // used). A token with no routed pick reads nothing.
  uint64_t row[MAXK];
  bool routed[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const int s = rs.slot[k];    // past topk: never read as a slot
    const int e = rs.expert[k];
    routed[k] = k < P.topk && s >= 0;
    row[k] = (uint64_t)(routed[k] ? e : 0) * (uint64_t)P.max_tokens + (uint64_t)(routed[k] ? s : 0);
  }
  bool any = false;
  uint64_t fallback = 0;
#pragma unroll
  for (int k = MAXK - 1; k >= 0; --k) {
    fallback = routed[k] ? row[k] : fallback;
    any = any || routed[k];
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  if (any) {
    uint4 v[MAXK];
    float wk[MAXK];
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      v[k] = P.y[(routed[k] ? row[k] : fallback) * (uint64_t)chunks + c];
      wk[k] = P.w[(uint64_t)t * P.topk + (k < P.topk ? k : P.topk - 1)];
    }
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __builtin_fmaf(wk[k], __uint_as_float(q[j] << 16), acc[2 * j]);
        const float b = __builtin_fmaf(wk[k], __uint_as_float(q[j] & 0xFFFF0000u), acc[2 * j + 1]);
        acc[2 * j] = routed[k] ? a : acc[2 * j];
        acc[2 * j + 1] = routed[k] ? b : acc[2 * j + 1];
      }
    }
  }
  float4* o = P.out + (uint64_t)t * (uint64_t)(chunks * 2) + 2 * (uint64_t)c;
  o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int blocks = p.num_tokens > 0 ? p.num_tokens * p.slices : 1;
  if (p.topk <= 2)
    combine_kernel<2><<<blocks, kCombineBlock, 0, stream>>>(p);
  else if (p.topk <= 4)
    combine_kernel<4><<<blocks, kCombineBlock, 0, stream>>>(p);
  else if (p.topk <= 8)
    combine_kernel<8><<<blocks, kCombineBlock, 0, stream>>>(p);
  else
    combine_kernel<16><<<blocks, kCombineBlock, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace llmoe
