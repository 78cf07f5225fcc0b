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
//  - A workgroup (256 threads) takes a tile of consecutive tokens (usually
//    one) and a group of its destination rows; `groups` workgroups share a
//    tile (small batches: so that a launch has ~512 workgroups), each
//    loading the tile's rows of x (fp8: and quantizing them) while the
//    routing prologue (route.h) computes the tile's slots.
//  - Dispatches below 64 MiB (dispatch_direct_kernel): every thread writes
//    the chunks it loaded (fp8: their codes) straight from its registers
//    to each of its group's rows, with dword-aligned stores at the row's
//    own 4-byte phase; no LDS copy, no barrier before the stores.
//  - Larger dispatches (dispatch_kernel): the tile's messages are built in
//    LDS and the destination rows (the send row and one receive row per
//    routed pick) go out from there. With wavefront rows each row is
//    written whole by one wavefront; with group rows (bf16 messages shared
//    among several groups) every row of the group is written by all its
//    threads in turn, and the send row is split among the groups. Message
//    rows are 4 + 2h bytes apart, so a destination starts at any 4-byte
//    phase. These stores are aligned to the destination: 0-3 head dwords,
//    then whole 16-byte chunks, then 0-3 tail dwords; the LDS side absorbs
//    the phase (dword-granular LDS reads), and the chunks are dealt to
//    lanes by whole 128-byte cache lines (copy_row_wave).
//  - Either way a receive row belongs to one group, so that group's count
//    follows whole messages.
//  - Messages are written with device-coherent (write-through) stores.
//    Every wavefront waits for its own stores; after a workgroup barrier
//    wavefront 0 adds one per routed pick of the group to that expert's
//    signal word, all picks in one device-scope atomic instruction: a
//    release without an L2 write-back (which costs tens of microseconds
//    over a launch). The other set's signal words are zeroed by
//    workgroup 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layout.h"
#include "route.h"
#include "message.h"

namespace llmoe {

// fp32 -> OCP e4m3 ("e4m3fn") codes, round to nearest even, saturating to
// +-448; the infinities saturate and every NaN gives 0x7F. Four values per
// call, packed little-endian into one word. The conversion itself is the
// gfx950 instruction v_cvt_pk_fp8_f32 (OCP e4m3, round to nearest even) on
// inputs clamped to [-448, 448] first, so that nothing reaches its overflow
// handling; NaN inputs are patched to 0x7F afterwards (rare: a scalar branch
// skips the patch when no lane has one).
__device__ __forceinline__ uint32_t e4m3_code4(float p0, float p1, float p2, float p3) {
  const float c0 = __builtin_amdgcn_fmed3f(p0, -448.0f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(p1, -448.0f, 448.0f);
  const float c2 = __builtin_amdgcn_fmed3f(p2, -448.0f, 448.0f);
  const float c3 = __builtin_amdgcn_fmed3f(p3, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
  uint32_t code = (uint32_t)w;
  const bool n0 = p0 != p0, n1 = p1 != p1, n2 = p2 != p2, n3 = p3 != p3;
  if (__builtin_expect(n0 || n1 || n2 || n3, 0)) {
    const uint32_t m = (n0 ? 0xFFu : 0u) | (n1 ? 0xFF00u : 0u) | (n2 ? 0xFF0000u : 0u) |
                       (n3 ? 0xFF000000u : 0u);
    code = (code & ~m) | (0x7F7F7F7Fu & m);
  }
  return code;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest bf16 magnitude among the 8 elements of a chunk, as its 15-bit
// pattern: magnitudes of numbers order like their bit patterns, and every
// NaN pattern (above 0x7F80, the infinity) is larger than all of them.
__device__ __forceinline__ uint32_t max_mag_bits(const u32x4 raw) {
  const u16x2 a = __builtin_bit_cast(u16x2, raw.x & 0x7FFF7FFFu);
  const u16x2 b = __builtin_bit_cast(u16x2, raw.y & 0x7FFF7FFFu);
  const u16x2 c = __builtin_bit_cast(u16x2, raw.z & 0x7FFF7FFFu);
  const u16x2 d = __builtin_bit_cast(u16x2, raw.w & 0x7FFF7FFFu);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
  return (uint32_t)(m.x > m.y ? m.x : m.y);
}

// The same with NaN elements left out (0 when all eight are NaN).
__device__ __forceinline__ uint32_t max_mag_bits_no_nan(const u32x4 raw) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t v = (w[k >> 1] >> (16 * (k & 1))) & 0x7FFFu;
    m = v <= 0x7F80u && v > m ? v : m;
  }
  return m;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t a) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, CTRL, 0xF, 0xF, false);
  return o > a ? o : a;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float a) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), CTRL, 0xF, 0xF, false));
}

// The same conversion without the clamp and the NaN patch, for inputs known
// to be numbers of magnitude below 464: v_cvt_pk_fp8_f32 rounds to nearest
// even and overflows only past 464, so it gives +-448 for everything in
// [448, 464] exactly as the clamped form does.
__device__ __forceinline__ uint32_t e4m3_code4_in_range(float p0, float p1, float p2, float p3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
  return (uint32_t)w;
}

// The eight codes of one unit (eight elements) of the fp8 message, given
// its block's inv. IN_RANGE: the products are known to be numbers below 464
// in magnitude (see quantize_plan).
template <bool IN_RANGE>
__device__ __forceinline__ uint2 quantize_codes(const u32x4 raw, float inv) {
  const float f[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                      bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
  if constexpr (IN_RANGE)
    return make_uint2(e4m3_code4_in_range(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                      e4m3_code4_in_range(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
  else
    return make_uint2(e4m3_code4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv),
                      e4m3_code4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv));
}

// Block inverses and scales of NS (1, 2 or 4) rounds of units, and whether
// the wavefront takes the conversion without clamp and NaN patch
// (wave-uniform).
struct QuantPlan {
  float inv[4];
  float scale[4];
  bool fast;
};

// The plan of NS rounds of units, u0 + s * blockDim for s < NS (all threads
// call it). A 128-element block is 16 consecutive lanes, one DPP row; the
// row reduces amax with four DPP steps (swap pairs, swap halves of quads,
// mirror halves of the row, mirror the row). The two divisions are then
// made once per lane instead of once per round: lane j of every quad
// divides for round j mod NS, and round s takes its block's inv and scale
// from lane s of the quad (DPP quad_perm [s,s,s,s]). Every lane of a row
// holds the same amax, so each quad has all NS.
template <int NS>
__device__ __forceinline__ QuantPlan quantize_plan(const u32x4 (&raw)[NS]) {
  static_assert(NS == 1 || NS == 2 || NS == 4, "rounds per quad lane");
  uint32_t m[NS];
  uint32_t mm = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = max_mag_bits(raw[s]);
    mm = m[s] > mm ? m[s] : mm;
  }
  if (__builtin_expect(__ballot(mm > 0x7F80u) != 0, 0)) {  // a NaN in the wave: rare
#pragma unroll
    for (int s = 0; s < NS; ++s) m[s] = max_mag_bits_no_nan(raw[s]);
  }
  float amax[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    uint32_t v = m[s];
    v = dpp_umax<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_umax<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_umax<0x141>(v);  // row_half_mirror
    v = dpp_umax<0x140>(v);  // row_mirror
    amax[s] = __uint_as_float(v << 16);
  }
  const int j = threadIdx.x & (NS - 1);
  float a = amax[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) a = j == s ? amax[s] : a;
  float inv = 0.0f, scale = 0.0f;
  if (a > 0.0f) {
    inv = 448.0f / a;
    scale = a / 448.0f;
  }
  QuantPlan p;
  p.inv[0] = dpp_f32<0x00>(inv);
  p.scale[0] = dpp_f32<0x00>(scale);
  if constexpr (NS > 1) {
    p.inv[1] = dpp_f32<0x55>(inv);
    p.scale[1] = dpp_f32<0x55>(scale);
  }
  if constexpr (NS > 2) {
    p.inv[2] = dpp_f32<0xAA>(inv);
    p.inv[3] = dpp_f32<0xFF>(inv);
    p.scale[2] = dpp_f32<0xAA>(scale);
    p.scale[3] = dpp_f32<0xFF>(scale);
  }
  // A block with a finite amax, a finite inv and no NaN in this lane gives
  // products of magnitude at most 448 * (1 + 2^-23): every |x| <= amax and
  // inv is 448 / amax rounded once. Such waves skip the clamp and the NaN
  // patch; a wave with any other block keeps them.
  bool special = mm > 0x7F80u;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    special = special || amax[s] == __builtin_inff() || p.inv[s] == __builtin_inff();
  p.fast = __ballot(special) == 0;
  return p;
}

// Codes of round s of a plan (wave-uniform choice of the encoder form).
__device__ __forceinline__ uint2 quantize_round_codes(const u32x4 raw, const QuantPlan& p, int s) {
  return __builtin_expect(p.fast, 1) ? quantize_codes<true>(raw, p.inv[s])
                                     : quantize_codes<false>(raw, p.inv[s]);
}

// Round s of a plan into an LDS message: unit u0 + s * blockDim (if below
// the row's units), its codes and, from the block's first unit, its scale.
__device__ __forceinline__ void quantize_round(uint8_t* msg, int hidden, int u0, int s,
                                               const u32x4 raw, const QuantPlan& p) {
  const int u = u0 + s * (int)blockDim.x;
  if (u >= hidden / 8) return;
  *reinterpret_cast<uint2*>(msg + 4 + 8 * u) = quantize_round_codes(raw, p, s);
  if ((u & 15) == 0) *reinterpret_cast<float*>(msg + 4 + hidden + 4 * (u >> 4)) = p.scale[s];
}

// NS rounds of units quantized into registers: codes of unit
// u0 + s * blockDim in code[s], its block's scale in scale[s] (all threads
// call it; units past the end are computed and not used).
template <int NS>
struct Fp8Regs {
  uint2 code[NS];
  float scale[NS];
};
template <int NS>
__device__ __forceinline__ Fp8Regs<NS> quantize_regs(const u32x4 (&raw)[NS]) {
  const QuantPlan p = quantize_plan<NS>(raw);
  Fp8Regs<NS> q;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    q.code[s] = quantize_round_codes(raw[s], p, s);
    q.scale[s] = p.scale[s];
  }
  return q;
}

// Four rounds of units, u0 + s * blockDim for s = 0..3 (all threads call
// it; units past the end are computed and not stored).
__device__ __forceinline__ void quantize_rounds(uint8_t* msg, int hidden, int u0,
                                                const u32x4 (&raw)[4]) {
  const QuantPlan p = quantize_plan<4>(raw);
#pragma unroll
  for (int s = 0; s < 4; ++s) quantize_round(msg, hidden, u0, s, raw[s], p);
}

// fp8 message body: per 128-element block, amax over the block (NaN
// ignored), inv = 448 / amax and scale = amax / 448 (correctly rounded fp32
// divisions; both 0 when amax is 0), codes e4m3(x * inv), scales after the
// codes. Each thread takes 8 elements per round, four rounds at a time;
// every thread runs every round (hidden % 128 == 0 and the block size is a
// multiple of 64, so a 16-lane row is wholly inside or outside the row of
// x). r holds the first four rounds' loads.
template <int NSTAGE>
__device__ __forceinline__ void stage_fp8(uint8_t* msg, const u32x4* __restrict__ xr, int hidden,
                                          const u32x4 (&r)[NSTAGE]) {
  static_assert(NSTAGE == 4, "one DPP quad lane per round");
  const int units = hidden / 8;
  const int B = blockDim.x;
  quantize_rounds(msg, hidden, threadIdx.x, r);
  for (int base = NSTAGE * B; base < units; base += NSTAGE * B) {  // uniform
    const int u0 = base + threadIdx.x;
    u32x4 q[NSTAGE];
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s) {
      const int u = u0 + s * B;
      q[s] = __builtin_nontemporal_load(xr + (u < units ? u : units - 1));
    }
    quantize_rounds(msg, hidden, u0, q);
  }
}

// message(t) into an LDS buffer: header, then the bf16 row or its fp8 form.
// r holds the row's first round of loads; further rounds (rows wider than
// 8192 columns) are read with non-temporal loads, as the first.
template <int DT, int NSTAGE>
__device__ __forceinline__ void build_message(uint8_t* msg, int t, const u32x4* __restrict__ xr,
                                              int hidden, const u32x4 (&r)[NSTAGE]) {
  const int tid = threadIdx.x;
  const int B = blockDim.x;
  const int chunks = hidden / 8;
  if (tid == 0) *reinterpret_cast<int32_t*>(msg) = t;
  if (DT == kBf16) {
#pragma unroll
    for (int u = 0; u < NSTAGE; ++u) {
      const int j = tid + u * B;
      if (j < chunks) *reinterpret_cast<u32x4*>(msg + 4 + 16 * j) = r[u];
    }
    for (int j0 = tid + NSTAGE * B; j0 < chunks; j0 += NSTAGE * B) {
      u32x4 q[NSTAGE];
#pragma unroll
      for (int u = 0; u < NSTAGE; ++u) {
        const int j = j0 + u * B;
        q[u] = __builtin_nontemporal_load(xr + (j < chunks ? j : chunks - 1));
      }
#pragma unroll
      for (int u = 0; u < NSTAGE; ++u) {
        const int j = j0 + u * B;
        if (j < chunks) *reinterpret_cast<u32x4*>(msg + 4 + 16 * j) = q[u];
      }
    }
  } else {
    stage_fp8<NSTAGE>(msg, xr, hidden, r);
  }
}

template <int DT, int VEC, bool GROUP_ROWS>
__global__ void __launch_bounds__(kDispatchBlock) dispatch_kernel(const DispatchParams P) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  __shared__ RouteShared rs;

  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += kDispatchBlock) P.sig_other[e] = 0;

  // workgroup -> (tile of tokens [t0, t1), row group g). Workgroups are
  // dealt to the 8 XCDs round-robin by index; all groups of one tile go to
  // the same XCD, so the tile's rows of x come from HBM once and the other
  // groups read them from that XCD's L2.
  const int xcd = blockIdx.x % kXcds;
  const int pos = blockIdx.x / kXcds;
  const int tile = xcd + kXcds * (pos / P.groups);
  const int g = pos - (pos / P.groups) * P.groups;
  const int t0 = tile * P.tile;
  if (t0 >= P.num_tokens) return;
  const int t1 = t0 + P.tile < P.num_tokens ? t0 + P.tile : P.num_tokens;
  const int K = P.topk;
  const int G = P.groups;
  const int chunks = P.hidden / 8;
  const uint32_t md = P.msg_bytes;
  const u32x4* x = reinterpret_cast<const u32x4*>(P.x);
  auto message_buffer = [&](int i) { return lds_raw + i * P.msg_stride + kMsgLdsOffset; };
  const int wave = tid / kWave;
  constexpr int kWaves = kDispatchBlock / kWave;

  // Destination rows of the tile: row rho = i * (K + 1) + m of token t0 + i
  // is its send row (m = 0) or the receive row of pick m - 1. Rows by
  // wavefront (GROUP_ROWS false): group g takes the rows rho = g,
  // g + groups, ..., and of those wavefront w every kWaves-th from the
  // w-th, each written whole by that wavefront. Rows by group (GROUP_ROWS):
  // group g takes part g of groups of every send row and the whole receive
  // rows of the picks m - 1 = g, g + groups, ..., each row written by all
  // its threads. Either way a receive row belongs to one group, so a count
  // raised by that group follows whole messages.
  auto owns_pick = [&](int i, int k) {
    const int rho = GROUP_ROWS ? k : i * (K + 1) + k + 1;
    return rho - (rho / G) * G == g;
  };

  // 1. the routing prologue; the loads of x[t0] go out with its first
  //    loads, and message(t0) is built in LDS once they are back, before
  //    the prologue's last barrier. Every wavefront then holds the tile's
  //    slots in its own lanes.
  constexpr int kStage = 4;
  u32x4 r[kStage];
  // A bf16 send row that one group writes whole and that fits one round of
  // registers goes out straight from them as soon as x[t0] is back, before
  // the routing histogram: the stores start while the prologue runs (1024
  // tokens of 7168 columns: 26.3 against 26.6 us).
  constexpr bool kEarlyKind = DT == kBf16 && !GROUP_ROWS;
  const bool early = kEarlyKind && G == 1 && chunks <= kStage * kDispatchBlock;
  // x is read with non-temporal loads: each row is read once here, and
  // loads that do not allocate leave the caches to the rows being written
  // (1024 tokens of 7168 columns: 24.3 against 26.3 us)
  const int wslot = route_tile<VEC, true>(
      P.idx, t0, t1, K, P.num_experts, P.max_tokens, rs,
      reinterpret_cast<int*>(lds_raw + P.tile * P.msg_stride), hist_cap_for(P.num_experts),
      [&]() {
        load_row<kStage, true>(r, x + (size_t)t0 * chunks, chunks);
        if constexpr (kEarlyKind) {
          if (early) {
            const BufRsrc sr = message_rsrc(P.send + (uint64_t)t0 * md, md);
            if (tid == 0) store_b32((uint32_t)t0, sr, 0);
            put_chunks<kStage, kDispatchBlock>(sr, r, 0, 0, chunks);
          }
        }
      },
      [&]() {
        build_message<DT, kStage>(message_buffer(0), t0, x + (size_t)t0 * chunks, P.hidden, r);
      });
  if (t1 - t0 > 1) {  // uniform: the tile's further messages, then one barrier
    for (int t = t0 + 1; t < t1; ++t) {
      load_row<kStage, true>(r, x + (size_t)t * chunks, chunks);
      build_message<DT, kStage>(message_buffer(t - t0), t, x + (size_t)t * chunks, P.hidden, r);
    }
    __syncthreads();
  }

  // 2. the rows
  if constexpr (GROUP_ROWS) {
    for (int i = 0; i < t1 - t0; ++i) {
      const uint8_t* msg = message_buffer(i);
      copy_message<true>(P.send + (uint64_t)(t0 + i) * md, msg, md, g, G);
      for (int k = g; k < K; k += G) {
        const int j = i * K + k;
        const int s = __builtin_amdgcn_readlane(wslot, j);
        if (s < 0) continue;  // masked
        copy_message<true>(
            P.recv + ((uint64_t)rs.expert[j] * (uint64_t)P.max_tokens + (uint64_t)s) * md, msg, md);
      }
    }
  } else {
    const int rows = (t1 - t0) * (K + 1);
    for (int rho = g + G * wave; rho < rows; rho += G * kWaves) {  // uniform per wavefront
      const int i = rho / (K + 1);
      const int m = rho - i * (K + 1);
      if (m == 0) {
        if (early && i == 0) continue;  // went out from registers
        copy_row_wave<true>(P.send + (uint64_t)(t0 + i) * md, message_buffer(i), md);
      } else {
        const int j = i * K + m - 1;
        const int s = __builtin_amdgcn_readlane(wslot, j);
        if (s < 0) continue;  // masked
        copy_row_wave<true>(
            P.recv + ((uint64_t)rs.expert[j] * (uint64_t)P.max_tokens + (uint64_t)s) * md,
            message_buffer(i), md);
      }
    }
  }

  // 3. publish: every wave waits until its own device-coherent stores are
  //    complete; after the barrier all of this group's messages are visible
  //    at device scope, and wavefront 0 adds one per routed pick of the
  //    group to that expert's signal word, all in one device-scope atomic
  //    instruction (lane j: entry j of the tile). The messages were written
  //    with device-coherent stores that have all completed, so the adds
  //    need no cache write-back of their own: a reader that loads the count
  //    with acquire semantics at device scope (which invalidates its L2
  //    copy) sees the messages. One instruction for the whole group matters
  //    when experts share a signal line: the lanes that name one line go to
  //    memory together, where one instruction per pick puts each add on the
  //    contended line alone (a batch of 128 tokens over 8 experts, whose
  //    words share one line, dispatched in 4.6 us against 6.3).
  //    The add is a 32-bit atomic on the word's low half (little-endian): a
  //    set's words start at 0 and a dispatch adds at most num_tokens * topk
  //    < 2^31, so no carry reaches the high half.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid < (t1 - t0) * K) {  // wavefront 0: tile * topk <= 64 entries
    const int i = tid / K;
    if (owns_pick(i, tid - i * K) && wslot >= 0)
      __hip_atomic_fetch_add(reinterpret_cast<unsigned int*>(P.sig + rs.expert[tid]), 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The dispatch with rows straight from registers, for dispatches below
// the whole-line size (their rows stay in L2 and MALL). Every thread keeps
// the 16-byte chunks of x it loaded (fp8: their codes and block scales) in
// registers and writes them to each of its group's rows itself: payload
// chunk u of a row at byte 4 + 16u (bf16) or codes at 4 + 8u and the block
// scale after the codes (fp8), dword-aligned buffer stores at whatever
// 4-byte phase the row has. There is no LDS copy of the message and no
// barrier before the stores; a receive row's stores start as soon as the
// slots are known, and the send row (bf16) goes out during the routing
// prologue. (128 tokens of 7168 columns dispatched in 5.51 us against 5.89
// through LDS, fp8 5.48 against 5.61, 512 tokens of 4096 columns 12.2
// against 12.8; for rows that go to HBM the straddled 128-byte lines cost
// more than the LDS round trip: the stores alone of 1024 such tokens took
// 24.5 us against 21.7 with whole-line stores, so large dispatches keep
// dispatch_kernel. Workgroups of 512 or 1024 threads, fewer rounds of
// quantization per thread, measured no faster.)
//
// Rows: group g of a tile writes the receive rows of the picks k = g,
// g + groups, ... and part g of groups of every send row (whole 128-element
// blocks for fp8, with their scales), each row by all its threads, so a
// count raised by the group follows whole messages. Tokens of a tile, and
// rows wider than one round of 4 * 256 chunks, go round by round; each
// round's loads are issued before the previous round's stores.
template <int DT, int VEC, int BLOCK>
__global__ void __launch_bounds__(BLOCK) dispatch_direct_kernel(const DispatchParams P) {
  extern __shared__ int hist[];  // hist_cap_for(num_experts) ints
  __shared__ RouteShared rs;

  const int tid = threadIdx.x;
  if (blockIdx.x == 0)
    for (int e = tid; e < P.num_experts; e += BLOCK) P.sig_other[e] = 0;

  // workgroup -> (tile of tokens [t0, t1), row group g), as dispatch_kernel
  const int xcd = blockIdx.x % kXcds;
  const int pos = blockIdx.x / kXcds;
  const int tile = xcd + kXcds * (pos / P.groups);
  const int g = pos - (pos / P.groups) * P.groups;
  const int t0 = tile * P.tile;
  if (t0 >= P.num_tokens) return;
  const int t1 = t0 + P.tile < P.num_tokens ? t0 + P.tile : P.num_tokens;
  const int K = P.topk;
  const int G = P.groups;
  const int units = P.hidden / 8;  // 16-byte chunks of x (fp8: 8-byte code groups)
  const uint32_t md = P.msg_bytes;
  const u32x4* x = reinterpret_cast<const u32x4*>(P.x);
  // the group's part of the send row, in units
  const int gran = DT == kBf16 ? 1 : 16;
  const int parts = units / gran;
  const int lo = gran * (parts * g / G);
  const int hi = gran * (parts * (g + 1) / G);

  // units per thread and round: 1024 units (8192 columns) per round
  constexpr int kStage = BLOCK == 256 ? 4 : BLOCK == 512 ? 2 : 1;
  static_assert(kStage * BLOCK == 1024, "workgroups of 256, 512 or 1024 threads");
  constexpr int kRound = kStage * BLOCK;
  u32x4 r[kStage];
  Fp8Regs<kStage> q;

  // this thread's units of one round into a row
  auto put_units = [&](BufRsrc rsrc, int base, int ulo, int uhi) {
    if constexpr (DT == kBf16) {
      put_chunks<kStage, BLOCK>(rsrc, r, base, ulo, uhi);
    } else {
#pragma unroll
      for (int s = 0; s < kStage; ++s) {
        const int u = base + tid + s * BLOCK;
        if (u < ulo || u >= uhi) continue;
        store_b64(q.code[s], rsrc, 4u + 8u * (uint32_t)u);
        if ((u & 15) == 0)
          store_b32(__float_as_uint(q.scale[s]), rsrc,
                    4u + (uint32_t)P.hidden + 4u * (uint32_t)(u >> 4));
      }
    }
  };
  // one 16-byte routing load per thread and round (single entries: 8)
  const int wslot = route_tile<VEC, true, VEC == 4 ? 1 : 8>(
      P.idx, t0, t1, K, P.num_experts, P.max_tokens, rs, hist, hist_cap_for(P.num_experts),
      [&]() { load_row<kStage>(r, x + (size_t)t0 * units, units); },
      [&]() {
        if constexpr (DT == kFp8) {
          q = quantize_regs<kStage>(r);
        } else {
          // the send row needs no slots: its part goes out while the
          // prologue's barrier waits (128 tokens of 7168 columns: 5.39
          // against 5.54 us; for fp8 the stores wait behind the
          // quantization and come out later, 5.61 against 5.50)
          const BufRsrc sr0 = message_rsrc(P.send + (uint64_t)t0 * md, md);
          if (g == 0 && tid == 0) store_b32((uint32_t)t0, sr0, 0);
          put_units(sr0, 0, lo, hi);
        }
      });

  int i = 0;
  int base = 0;
  while (true) {  // uniform: one (token, round) per pass
    int ni = i, nbase = base + kRound;
    if (nbase >= units) {
      ni = i + 1;
      nbase = 0;
    }
    const bool more = t0 + ni < t1;
    u32x4 nx[kStage];
    if (more) load_row<kStage>(nx, x + (size_t)(t0 + ni) * units, units, nbase);

    const int t = t0 + i;
    const BufRsrc sr = message_rsrc(P.send + (uint64_t)t * md, md);
    if (DT == kFp8 || i > 0 || base > 0) {  // bf16: the first round went out above
      if (base == 0 && g == 0 && tid == 0) store_b32((uint32_t)t, sr, 0);
      put_units(sr, base, lo, hi);
    }
    for (int k = g; k < K; k += G) {
      const int j = i * K + k;
      const int slot = __builtin_amdgcn_readlane(wslot, j);
      if (slot < 0) continue;  // masked
      const BufRsrc rr = message_rsrc(
          P.recv + ((uint64_t)rs.expert[j] * (uint64_t)P.max_tokens + (uint64_t)slot) * md, md);
      if (base == 0 && tid == 0) store_b32((uint32_t)t, rr, 0);
      put_units(rr, base, 0, units);
    }
    if (!more) break;
#pragma unroll
    for (int s = 0; s < kStage; ++s) r[s] = nx[s];
    if constexpr (DT == kFp8) q = quantize_regs<kStage>(r);
    i = ni;
    base = nbase;
  }

  // publish, as dispatch_kernel: every wave's stores complete, one barrier,
  // then wavefront 0 adds the group's picks in one device-scope atomic
  // instruction
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid < (t1 - t0) * K) {  // wavefront 0: tile * topk <= 64 entries
    const int k = tid - (tid / K) * K;
    if (k - (k / G) * G == g && wslot >= 0)
      __hip_atomic_fetch_add(reinterpret_cast<unsigned int*>(P.sig + rs.expert[tid]), 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int DT, int VEC, int BLOCK>
static hipError_t launch_direct_block(const DispatchParams& p, hipStream_t stream) {
  const int tiles = p.num_tokens > 0 ? (p.num_tokens + p.tile - 1) / p.tile : 1;
  const int rounds = (tiles + kXcds - 1) / kXcds;
  const size_t lds = sizeof(int) * hist_cap_for(p.num_experts);
  dispatch_direct_kernel<DT, VEC, BLOCK><<<rounds * kXcds * p.groups, BLOCK, lds, stream>>>(p);
  return hipGetLastError();
}

template <int DT, int VEC>
static hipError_t launch_direct(const DispatchParams& p, hipStream_t stream) {
  return launch_direct_block<DT, VEC, kDispatchBlock>(p, stream);
}

template <int DT, int VEC, bool GROUP_ROWS>
static hipError_t launch_dt(const DispatchParams& p, hipStream_t stream) {
  const int tiles = p.num_tokens > 0 ? (p.num_tokens + p.tile - 1) / p.tile : 1;
  // whole rounds of kXcds tiles, so that the index mapping covers every tile
  const int rounds = (tiles + kXcds - 1) / kXcds;
  const size_t lds = (size_t)p.tile * p.msg_stride + sizeof(int) * hist_cap_for(p.num_experts);
  dispatch_kernel<DT, VEC, GROUP_ROWS>
      <<<rounds * kXcds * p.groups, kDispatchBlock, lds, stream>>>(p);
  return hipGetLastError();
}

template <int DT, bool GROUP_ROWS>
static hipError_t launch_lds(const DispatchParams& p, hipStream_t stream) {
  return p.wide_idx ? launch_dt<DT, 4, GROUP_ROWS>(p, stream)
                    : launch_dt<DT, 1, GROUP_ROWS>(p, stream);
}

// Below 64 MiB of rows the register-direct kernel; at 64 MiB or more the
// LDS kernel with whole-line stores.
template <int DT>
static hipError_t launch_modes(const DispatchParams& p, hipStream_t stream) {
  if (!p.line_align)
    return p.vec_idx ? launch_direct<DT, 4>(p, stream) : launch_direct<DT, 1>(p, stream);
  return p.group_rows ? launch_lds<DT, true>(p, stream) : launch_lds<DT, false>(p, stream);
}

hipError_t launch_dispatch(const DispatchParams& p, int dtype, hipStream_t stream) {
  return dtype == kBf16 ? launch_modes<kBf16>(p, stream) : launch_modes<kFp8>(p, stream);
}

// The fp8 encoders above, applied element-wise in groups of four; lets a
// test compare them with an independent encoder on chosen fp32 inputs.
// IN_RANGE runs the form ordinary fp8 waves use (no clamp, no NaN patch),
// whose codes are defined for numbers of magnitude at most 448 * (1 + 2^-23).
template <bool IN_RANGE>
__global__ void e4m3_probe_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                  uint64_t n) {
  const uint64_t groups = (n + 3) / 4;
  for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (uint64_t)gridDim.x * blockDim.x) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = 4 * g + j < n ? in[4 * g + j] : 0.0f;
    const uint32_t code = IN_RANGE ? e4m3_code4_in_range(v[0], v[1], v[2], v[3])
                                   : e4m3_code4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * g + j < n) out[4 * g + j] = (uint8_t)(code >> (8 * j));
  }
}

hipError_t launch_e4m3_probe(const float* in, uint8_t* out, uint64_t n, bool in_range,
                             hipStream_t stream) {
  uint64_t blocks = ((n + 3) / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  if (in_range)
    e4m3_probe_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(in, out, n);
  else
    e4m3_probe_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(in, out, n);
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
