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
// Design on gfx950: one workgroup per (tile of consecutive tokens, run of
// columns); the runs of a row are equal, one 16-byte chunk per thread
// (kernels.h, combine_shape). It computes the tile's slots once (route.h);
// then every thread issues its topk 16-byte loads of bf16 expert rows at
// once (a tile of two tokens: both tokens' loads), folds them with
// v_fma_f32 in k order, and writes 8 fp32 results per token as two 16-byte
// streaming stores (gather.h). Workgroup 0 zeroes the other set's signal
// words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"
#include "route.h"
#include "gather.h"

namespace llmoe {

template <int MAXK, bool STREAM, int VEC>
__global__ void __launch_bounds__(kCombineMaxBlock) combine_kernel(const CombineParams P) {
  __shared__ RouteShared rs;
  extern __shared__ int hist[];  // hist_cap_for(num_experts) ints
  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += (int)blockDim.x) P.sig_other[e] = 0;

  // workgroup -> (tile of tokens [t0, t1), run of columns sl)
  const int tile = blockIdx.x / P.slices;
  const int sl = blockIdx.x - tile * P.slices;
  const int t0 = tile * P.tile;
  if (t0 >= P.num_tokens) return;
  const int t1 = t0 + P.tile < P.num_tokens ? t0 + P.tile : P.num_tokens;

  // the tile's slots in LDS (wavefront 0 ranks them; a barrier shares
  // them), the table read by two 16-byte loads per thread and round (8
  // single-entry loads when it cannot be read 4 entries at a time). Every
  // wavefront ranking its own copy instead, which saves that barrier,
  // measured slower for large batches (1024 tokens of 7168 columns: 30.1
  // against 29.7 us) and no faster for small ones.
  route_tile<VEC, false, VEC == 4 ? 2 : 8>(P.idx, t0, t1, P.topk, P.num_experts, P.max_tokens,
                                           rs, hist, hist_cap_for(P.num_experts));

  const int chunks = P.hidden / 8;
  const int c = sl * (int)blockDim.x + tid;
  if (c >= chunks) return;
  // token i of the tile: its picks' rows from the tile's slots
  auto tok = [&](int i, uint64_t (&row)[MAXK], bool (&routed)[MAXK], float (&w)[MAXK]) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const int kk = k < P.topk ? k : 0;
      const int s = rs.slot[i * P.topk + kk];
      routed[k] = k < P.topk && s >= 0;
      row[k] = (uint64_t)(routed[k] ? rs.expert[i * P.topk + kk] : 0) * (uint64_t)P.max_tokens +
               (uint64_t)(routed[k] ? s : 0);
      w[k] = P.w[(uint64_t)(t0 + i) * P.topk + kk];
    }
  };
  auto out = [&](int i) {
    return reinterpret_cast<gf32x4*>(P.out) + (uint64_t)(t0 + i) * (uint64_t)(chunks * 2) +
           2 * (uint64_t)c;
  };
  gather_tile<MAXK, STREAM>(reinterpret_cast<const g32x4*>(P.y), t1 - t0, c, chunks, tok, out);
}

template <bool STREAM, int VEC>
static void launch_k(const CombineParams& p, int blocks, hipStream_t stream) {
  const size_t lds = sizeof(int) * hist_cap_for(p.num_experts);
  if (p.topk <= 2)
    combine_kernel<2, STREAM, VEC><<<blocks, p.block, lds, stream>>>(p);
  else if (p.topk <= 4)
    combine_kernel<4, STREAM, VEC><<<blocks, p.block, lds, stream>>>(p);
  else if (p.topk <= 8)
    combine_kernel<8, STREAM, VEC><<<blocks, p.block, lds, stream>>>(p);
  else
    combine_kernel<16, STREAM, VEC><<<blocks, p.block, lds, stream>>>(p);
}

template <bool STREAM>
static void launch_vec(const CombineParams& p, int blocks, hipStream_t stream) {
  if (p.vec_idx)
    launch_k<STREAM, 4>(p, blocks, stream);
  else
    launch_k<STREAM, 1>(p, blocks, stream);
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int tiles = p.num_tokens > 0 ? (p.num_tokens + p.tile - 1) / p.tile : 1;
  const int blocks = tiles * p.slices;
  if (p.stream_rows)
    launch_vec<true>(p, blocks, stream);
  else
    launch_vec<false>(p, blocks, stream);
  return hipGetLastError();
}

}  // namespace llmoe
