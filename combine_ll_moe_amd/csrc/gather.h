// The combine's gather-and-fold of one token over one thread's 8 columns,
// given the expert-output rows of its picks. Shared by the combine (rows
// from the routing prologue) and the gather-only measurement probe (rows
// handed in), so that the probe times exactly the combine's loads and fold.
//
// acc = fmaf(w[k], y[row[k]][c], acc) over the routed picks in ascending k,
// from +0.0f, in fp32: one fixed operand order, so every call forms the same
// expression and returns the same bits (memra-engine src/tp_ar.rs,
// memra_tp_ar_1stage: the inputs are read in one global order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmoe {

typedef uint32_t g32x4 __attribute__((ext_vector_type(4)));
typedef float gf32x4 __attribute__((ext_vector_type(4)));

// y: bf16 rows of `chunks` 16-byte chunks; column chunk c of each routed
// row is loaded (all MAXK loads issued before any is used), folded in k
// order, and the 8 fp32 results are written to o[0..1] with streaming
// stores. A pick that is not routed borrows a routed pick's row address so
// that every load is unconditional; its value is never used, and a token
// with no routed pick reads nothing and writes +0.0f.
template <int MAXK, bool STREAM>
__device__ __forceinline__ void gather_fold(const g32x4* __restrict__ y, const uint64_t (&row)[MAXK],
                                            const bool (&routed)[MAXK], const float (&w)[MAXK],
                                            int c, int chunks, gf32x4* o) {
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
    g32x4 v[MAXK];
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const g32x4* src = y + (routed[k] ? row[k] : fallback) * (uint64_t)chunks + c;
      v[k] = STREAM ? __builtin_nontemporal_load(src) : *src;
    }
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float a = __builtin_fmaf(w[k], __uint_as_float(q[h] << 16), acc[2 * h]);
        const float b = __builtin_fmaf(w[k], __uint_as_float(q[h] & 0xFFFF0000u), acc[2 * h + 1]);
        acc[2 * h] = routed[k] ? a : acc[2 * h];
        acc[2 * h + 1] = routed[k] ? b : acc[2 * h + 1];
      }
    }
  }
  // streaming (non-temporal) stores: the output is not read again here
  const gf32x4 lo = {acc[0], acc[1], acc[2], acc[3]};
  const gf32x4 hi = {acc[4], acc[5], acc[6], acc[7]};
  __builtin_nontemporal_store(lo, o);
  __builtin_nontemporal_store(hi, o + 1);
}

}  // namespace llmoe
