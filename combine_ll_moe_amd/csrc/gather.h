// The combine's gather-and-fold of a tile's tokens over one thread's 8
// columns, given the expert-output rows of their picks. Shared by the
// combine (rows from the routing prologue) and the gather-only measurement
// probe (rows handed in), so that the probe times exactly the combine's
// loads and fold.
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

// The fold of NT tokens' loaded chunks: token i's pick k contributes
// v[i][k] (8 bf16 columns) with weight w[i][k] when routed[i][k], in k order
// from +0.0f; the 8 fp32 results go to o(i)[0..1] with streaming
// (non-temporal) stores, the output not being read again here. Picks that
// are not routed leave the sum as it is, whatever their v holds.
template <int NT, int MAXK, typename Out>
__device__ __forceinline__ void fold_store(const g32x4 (&v)[NT][MAXK],
                                           const bool (&routed)[NT][MAXK],
                                           const float (&w)[NT][MAXK], const Out& o) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const uint32_t q[4] = {v[i][k].x, v[i][k].y, v[i][k].z, v[i][k].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float a = __builtin_fmaf(w[i][k], __uint_as_float(q[h] << 16), acc[2 * h]);
        const float b =
            __builtin_fmaf(w[i][k], __uint_as_float(q[h] & 0xFFFF0000u), acc[2 * h + 1]);
        acc[2 * h] = routed[i][k] ? a : acc[2 * h];
        acc[2 * h + 1] = routed[i][k] ? b : acc[2 * h + 1];
      }
    }
    gf32x4* out = o(i);
    const gf32x4 lo = {acc[0], acc[1], acc[2], acc[3]};
    const gf32x4 hi = {acc[4], acc[5], acc[6], acc[7]};
    __builtin_nontemporal_store(lo, out);
    __builtin_nontemporal_store(hi, out + 1);
  }
}

// Column chunk c of each routed pick's row of NT tokens (token i's rows,
// routing flags and weights from tok(i, row, routed, w)), every load issued
// before any is used, then folded and stored by fold_store. A pick that is not routed
// borrows a routed pick's row address of its token (row 0 when none is
// routed, so y must have a row) so that every load is unconditional and no
// branch stands between the loads; its value is never used, and a token
// with no routed pick writes +0.0f. y: bf16 rows of `chunks` 16-byte
// chunks.
template <int NT, int MAXK, bool STREAM, typename Tok, typename Out>
__device__ __forceinline__ void gather_fold(const g32x4* __restrict__ y, int t_first, int c,
                                            int chunks, const Tok& tok, const Out& o) {
  bool routed[NT][MAXK];
  float w[NT][MAXK];
  g32x4 v[NT][MAXK];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    uint64_t row[MAXK];
    tok(t_first + i, row, routed[i], w[i]);
    uint64_t fallback = 0;
#pragma unroll
    for (int k = MAXK - 1; k >= 0; --k) fallback = routed[i][k] ? row[k] : fallback;
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      const g32x4* src = y + (routed[i][k] ? row[k] : fallback) * (uint64_t)chunks + c;
      v[i][k] = STREAM ? __builtin_nontemporal_load(src) : *src;
    }
  }
  fold_store<NT, MAXK>(v, routed, w, [&](int i) { return o(t_first + i); });
}

// A tile's tokens (at most two): with at most 8 picks both tokens' loads go
// out before either is folded (1024 tokens of 7168 columns: combine 28.1
// against 28.9 us one token after the other, 16 loads of 16 bytes in flight
// per lane); with more picks, or one token, token by token. tok(i, row,
// routed, w) fills token i's rows, routing flags and weights; o(i) is token
// i's output at column chunk c.
template <int MAXK, bool STREAM, typename Tok, typename Out>
__device__ __forceinline__ void gather_tile(const g32x4* __restrict__ y, int n, int c, int chunks,
                                            const Tok& tok, const Out& o) {
  if (MAXK <= 8 && n == 2) {
    gather_fold<2, MAXK, STREAM>(y, 0, c, chunks, tok, o);
  } else {
    for (int i = 0; i < n; ++i) gather_fold<1, MAXK, STREAM>(y, i, c, chunks, tok, o);
  }
}

}  // namespace llmoe
