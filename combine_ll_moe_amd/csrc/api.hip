// C ABI of libllmoe.so (declared in include/ll_moe.h): argument checks,
// layout offsets, launch shape, and the launch on the caller's stream.
// Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ll_moe.h"
#include "ll_moe_diag.h"
#include "expert.h"
#include "kernels.h"
#include "layout.h"
#include "route.h"

using namespace llmoe;

namespace {

// Launch shapes (the shared constants are in kernels.h). Dispatch: a
// workgroup takes a tile of consecutive tokens and every groups-th message
// of each; combine: a tile of tokens and one run of columns.
//
// The dispatch keeps one token per workgroup up to twice as many
// workgroups: a batch of 1024 tokens of 7168 columns dispatches 7% faster
// with 1024 one-token workgroups (four resident per CU) than with 512
// two-token ones, whose second message waits behind the first.
constexpr int kDispatchTileBlocks = 1024;
// LDS a dispatch workgroup may use for message buffers: 64 KiB less the
// routing prologue's share (its tile entries and its histogram).
uint32_t dispatch_lds_budget(int num_experts) {
  return 65536u - (uint32_t)sizeof(RouteShared) - 4u * (uint32_t)hist_cap_for(num_experts);
}

// The routing prologues read the table 4 entries per 16-byte load when it
// is 16-byte aligned and a whole number of 4-entry vectors (vec_idx), with
// few loads per thread and round: one in the register-path dispatch (128
// tokens of 7168 columns: 5.18 against 5.40 us with 8 single-entry loads;
// 512 tokens of 4096 columns, three rounds: 11.60 against 11.95; 2048
// tokens of 1024 columns, sixteen rounds: 16.0 against 16.3 with 8 loads of
// 4 entries), two in
// the combine (128 tokens of 7168 columns, step 10.12 against 10.36 us with
// both changes). The dispatch of 64 MiB or more reads 8 vectors per thread
// and round, but only for tables of more than 4096 entries (wide_idx), so
// that a late tile's later rounds do not queue behind the other
// workgroups' message stores (1024 tokens of 8 picks: prologues of up to
// 9 us; dispatch 28.9 -> 28.0 us); fewer loads per round measured slower
// there (25.4 us with one, 24.7 with two, 24.4 with four or eight).
constexpr int64_t kWideIdxEntries = 4096;

int vec_idx_for(const int32_t* idx, int num_tokens, int topk) {
  const int64_t entries = (int64_t)num_tokens * topk;
  return entries % 4 == 0 && ((uintptr_t)idx & 15) == 0;
}

int wide_idx_for(const int32_t* idx, int num_tokens, int topk) {
  return (int64_t)num_tokens * topk > kWideIdxEntries && vec_idx_for(idx, num_tokens, topk);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_shape(int max_tokens, int num_tokens, int hidden, int num_experts, int topk,
                int dtype, int parity, Layout* L) {
  if (parity != 0 && parity != 1) return LL_MOE_INVALID_ARGUMENT;
  if (!make_layout(max_tokens, hidden, num_experts, dtype, L)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens) return LL_MOE_INVALID_ARGUMENT;
  if (topk < 1 || topk > num_experts || topk > LL_MOE_MAX_TOPK) return LL_MOE_INVALID_ARGUMENT;
  if (dtype == kBf16 && hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (L->dispatch_msg > kMaxMessageBytes) return LL_MOE_INVALID_ARGUMENT;
  if (num_experts > LL_MOE_MAX_EXPERTS) return LL_MOE_INVALID_ARGUMENT;
  // slot rows and token offsets are formed in 64 bits, entry indices in 32
  if ((int64_t)max_tokens * topk > INT32_MAX) return LL_MOE_INVALID_ARGUMENT;
  return LL_MOE_SUCCESS;
}

int from_hip(hipError_t e) { return e == hipSuccess ? LL_MOE_SUCCESS : LL_MOE_HIP_ERROR; }

}  // namespace

extern "C" int ll_moe_layout_bytes(int max_tokens, int hidden, int num_experts, int dtype,
                                   size_t* out_bytes) {
  Layout L;
  if (!out_bytes || !make_layout(max_tokens, hidden, num_experts, dtype, &L))
    return LL_MOE_INVALID_ARGUMENT;
  *out_bytes = (size_t)L.total;
  return LL_MOE_SUCCESS;
}

extern "C" int ll_moe_layout_offsets(int max_tokens, int hidden, int num_experts, int dtype,
                                     int parity, size_t* send_off, size_t* recv_off,
                                     size_t* sig_off, size_t* msg_bytes) {
  Layout L;
  if (!send_off || !recv_off || !sig_off || (parity != 0 && parity != 1) ||
      !make_layout(max_tokens, hidden, num_experts, dtype, &L))
    return LL_MOE_INVALID_ARGUMENT;
  *send_off = (size_t)L.send_off(parity);
  *recv_off = (size_t)L.recv_off(parity);
  *sig_off = (size_t)L.sig_off(parity);
  if (msg_bytes) *msg_bytes = (size_t)L.dispatch_msg;
  return LL_MOE_SUCCESS;
}

extern "C" int ll_moe_dispatch(void* layout, int max_tokens, int num_tokens, int hidden,
                               int num_experts, int topk, int dtype, int parity, const void* x,
                               const int32_t* topk_idx, hipStream_t stream) {
  Layout L;
  int rc = check_shape(max_tokens, num_tokens, hidden, num_experts, topk, dtype, parity, &L);
  if (rc != LL_MOE_SUCCESS) return rc;
  if (!layout || !aligned(layout, 16)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens > 0 && (!x || !topk_idx || !aligned(x, 16) || !aligned(topk_idx, 4)))
    return LL_MOE_INVALID_ARGUMENT;

  uint8_t* base = static_cast<uint8_t*>(layout);
  DispatchParams p;
  p.send = base + L.send_off(parity);
  p.recv = base + L.recv_off(parity);
  p.sig = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity));
  p.sig_other = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity ^ 1));
  p.x = static_cast<const uint4*>(x);
  p.idx = topk_idx;
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.topk = topk;
  // Launch shape: 256-thread workgroups, one token per workgroup up to
  // kDispatchTileBlocks of them, then two. A small batch shares each token's
  // rows among `groups` workgroups, so that the launch has ~512 workgroups:
  // each loads (fp8: quantizes) the whole row of x and writes its rows. A
  // group needs at least two rows: more groups than that add atomic
  // instructions on the signal lines (128 tokens over 8 experts, whose
  // words share one line: 6.0 us with two rows per group against 4.6 with
  // three); with rows from registers 4 groups stay best for 128 tokens of
  // 7168 columns (bf16 5.51 us against 5.66 with 2 or 3, fp8 5.48 against
  // 5.53-5.56). Dispatches of 64 MiB or more build the messages in LDS;
  // their rows go out by wavefront (each written whole by one wavefront),
  // except for bf16 messages shared among groups, which go out by group
  // (each row by all the group's threads, the send row split among the
  // groups), measured 5.85 against 6.13 us through LDS for 128 tokens of
  // 7168 columns, where the fp8 message is the other way round (5.70
  // against 6.19).
  int groups = num_tokens > 0 ? kTargetBlocks / num_tokens : 1;
  if (groups > (topk + 1) / 2) groups = (topk + 1) / 2;
  p.groups = groups < 1 ? 1 : groups;
  p.group_rows = dtype == kBf16 && p.groups > 1;
  p.tile = tile_for(num_tokens, p.groups, topk, kDispatchTileBlocks);
  p.msg_bytes = (uint32_t)L.dispatch_msg;
  p.msg_stride = ((uint32_t)kMsgLdsOffset + p.msg_bytes + 15u) & ~15u;
  // every message of a tile sits in LDS at once
  if ((uint64_t)p.tile * p.msg_stride > dispatch_lds_budget(num_experts)) p.tile = 1;
  // Large dispatches write mostly to HBM, where aligned whole-line stores
  // from LDS pay off; smaller ones stay in L2 and MALL, where stores straight
  // from registers at the rows' own phase are faster (see
  // dispatch_direct_kernel).
  p.line_align = (uint64_t)num_tokens * (uint64_t)(topk + 1) * L.dispatch_msg >= kStreamRowsBytes;
  p.vec_idx = vec_idx_for(topk_idx, num_tokens, topk);
  p.wide_idx = wide_idx_for(topk_idx, num_tokens, topk);
  return from_hip(launch_dispatch(p, dtype, stream));
}

extern "C" int ll_moe_combine(void* layout, int max_tokens, int num_tokens, int hidden,
                              int num_experts, int topk, int dtype, int parity,
                              const void* expert_out, const int32_t* topk_idx,
                              const float* topk_weights, float* out, hipStream_t stream) {
  Layout L;
  int rc = check_shape(max_tokens, num_tokens, hidden, num_experts, topk, dtype, parity, &L);
  if (rc != LL_MOE_SUCCESS) return rc;
  if (hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !aligned(layout, 16)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens > 0) {
    if (!expert_out || !topk_idx || !topk_weights || !out) return LL_MOE_INVALID_ARGUMENT;
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) ||
        !aligned(topk_weights, 4))
      return LL_MOE_INVALID_ARGUMENT;
    // out may not overlap the expert outputs
    const uintptr_t y0 = (uintptr_t)expert_out;
    const uintptr_t y1 = y0 + (uint64_t)num_experts * max_tokens * hidden * 2;
    const uintptr_t o0 = (uintptr_t)out;
    const uintptr_t o1 = o0 + (uint64_t)num_tokens * hidden * 4;
    if (o0 < y1 && y0 < o1) return LL_MOE_INVALID_ARGUMENT;
  }

  uint8_t* base = static_cast<uint8_t*>(layout);
  CombineParams p;
  p.sig_other = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity ^ 1));
  p.y = static_cast<const uint4*>(expert_out);
  p.idx = topk_idx;
  p.w = topk_weights;
  p.out = reinterpret_cast<float4*>(out);
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.topk = topk;
  // Large gathers stream past the caches: read with non-temporal loads they
  // leave L2 and MALL to the next dispatch's traffic (a whole step is ~20%
  // faster at 117 MB of rows); small ones gain from the cached path.
  p.stream_rows = (uint64_t)num_tokens * topk * hidden * 2 >= kStreamRowsBytes;
  const CombineShape shape = combine_shape(num_tokens, hidden, topk, p.stream_rows);
  p.slices = shape.slices;
  p.tile = shape.tile;
  p.block = shape.block;
  p.vec_idx = vec_idx_for(topk_idx, num_tokens, topk);
  return from_hip(launch_combine(p, stream));
}

namespace {

// Two-phase combine launch shape: the expert side spreads the received rows
// over a fixed grid (the host does not know how many there are); the token
// side takes the fused combine's shape.
constexpr int kSendBlocks = 1024;

int check_two_phase(const Layout& L, int hidden, int num_experts, int max_tokens, void* layout) {
  if (hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (num_experts > LL_MOE_SEND_MAX_EXPERTS) return LL_MOE_INVALID_ARGUMENT;
  if (L.combine_msg > kMaxMessageBytes) return LL_MOE_INVALID_ARGUMENT;
  if ((int64_t)num_experts * max_tokens > INT32_MAX) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !aligned(layout, 16)) return LL_MOE_INVALID_ARGUMENT;
  return LL_MOE_SUCCESS;
}

bool overlaps(const void* a, uint64_t a_bytes, const void* b, uint64_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

}  // namespace

extern "C" int ll_moe_combine_send(void* layout, int max_tokens, int hidden, int num_experts,
                                   int dtype, int parity, const void* expert_out,
                                   hipStream_t stream) {
  Layout L;
  int rc = check_shape(max_tokens, 0, hidden, num_experts, 1, dtype, parity, &L);
  if (rc != LL_MOE_SUCCESS) return rc;
  rc = check_two_phase(L, hidden, num_experts, max_tokens, layout);
  if (rc != LL_MOE_SUCCESS) return rc;
  if (!expert_out || !aligned(expert_out, 16)) return LL_MOE_INVALID_ARGUMENT;
  // the staging rows may not overlap the expert outputs they are copied from
  if (overlaps(layout, L.total, expert_out, (uint64_t)num_experts * max_tokens * hidden * 2))
    return LL_MOE_INVALID_ARGUMENT;

  uint8_t* base = static_cast<uint8_t*>(layout);
  SendParams p;
  p.sig = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity));
  p.sig_other = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity ^ 1));
  p.recv = base + L.recv_off(parity);
  p.stage = base + L.send_off(parity);
  p.y = static_cast<const uint4*>(expert_out);
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.msg_bytes = (uint32_t)L.dispatch_msg;
  p.comb_bytes = (uint32_t)L.combine_msg;
  // LDS: the count prefix, then one or two message buffers
  const uint32_t prefix_bytes = count_prefix_bytes(num_experts);
  const uint32_t stride = ((uint32_t)kMsgLdsOffset + p.comb_bytes + 15u) & ~15u;
  p.nbuf = prefix_bytes + 2 * stride <= 65536u - 64u ? 2 : 1;
  const int64_t most_rows = (int64_t)num_experts * max_tokens;
  const int blocks = most_rows < kSendBlocks ? (int)most_rows : kSendBlocks;
  return from_hip(launch_combine_send(p, blocks, stream));
}

extern "C" int ll_moe_combine_recv(void* layout, int max_tokens, int num_tokens, int hidden,
                                   int num_experts, int topk, int dtype, int parity,
                                   const int32_t* topk_idx, const float* topk_weights, float* out,
                                   int max_spins, int32_t* status, hipStream_t stream) {
  Layout L;
  int rc = check_shape(max_tokens, num_tokens, hidden, num_experts, topk, dtype, parity, &L);
  if (rc != LL_MOE_SUCCESS) return rc;
  rc = check_two_phase(L, hidden, num_experts, max_tokens, layout);
  if (rc != LL_MOE_SUCCESS) return rc;
  if (max_spins < 1) return LL_MOE_INVALID_ARGUMENT;
  if (!status || !aligned(status, 4)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens > 0) {
    if (!topk_idx || !topk_weights || !out) return LL_MOE_INVALID_ARGUMENT;
    if (!aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4))
      return LL_MOE_INVALID_ARGUMENT;
    // out may not overlap the layout whose staging rows it folds
    if (overlaps(layout, L.total, out, (uint64_t)num_tokens * hidden * 4))
      return LL_MOE_INVALID_ARGUMENT;
  }

  uint8_t* base = static_cast<uint8_t*>(layout);
  RecvParams p;
  p.sig = reinterpret_cast<const unsigned long long*>(base + L.sig_off(parity));
  p.sig_other = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity ^ 1));
  p.stage = base + L.send_off(parity);
  p.idx = topk_idx;
  p.w = topk_weights;
  p.out = reinterpret_cast<float4*>(out);
  p.status = status;
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.topk = topk;
  p.comb_bytes = (uint32_t)L.combine_msg;
  p.max_spins = max_spins;
  p.stream_rows = (uint64_t)num_tokens * topk * hidden * 2 >= kStreamRowsBytes;
  const CombineShape shape = combine_shape(num_tokens, hidden, topk, p.stream_rows);
  p.slices = shape.slices;
  p.tile = shape.tile;
  p.block = shape.block;
  return from_hip(launch_combine_recv(p, stream));
}

namespace {
// Expert side of the dispatch: a fixed grid, one workgroup per CU, so that
// while it waits beside a running dispatch it leaves the dispatch room; two
// per CU when the step routes 64 MiB of messages or more, whose copy is
// bandwidth-bound (1024 tokens of 7168 columns, measured with plain
// payload stores: unpack 44.6 against 48.7 us, and the dispatch with a
// receiver waiting beside it 81.3 against 86.3 us to the expert inputs;
// four per CU unpack no faster and slow that dispatch to 86.9).
constexpr int kUnpackBlocks = 256;
constexpr int kUnpackWideBlocks = 512;
}  // namespace

extern "C" int ll_moe_dispatch_recv(void* layout, int max_tokens, int hidden, int num_experts,
                                    int dtype, int parity, int expected, void* payload,
                                    float* scales, int32_t* src_tokens, int32_t* counts,
                                    int max_spins, int32_t* status, hipStream_t stream) {
  Layout L;
  int rc = check_shape(max_tokens, 0, hidden, num_experts, 1, dtype, parity, &L);
  if (rc != LL_MOE_SUCCESS) return rc;
  if (dtype == kBf16 && hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (num_experts > LL_MOE_SEND_MAX_EXPERTS) return LL_MOE_INVALID_ARGUMENT;
  const int64_t slots = (int64_t)num_experts * max_tokens;
  if (slots > INT32_MAX) return LL_MOE_INVALID_ARGUMENT;
  if (expected < 0 || expected > slots || max_spins < 1) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !aligned(layout, 16)) return LL_MOE_INVALID_ARGUMENT;
  if (!payload || !src_tokens || !counts || !status) return LL_MOE_INVALID_ARGUMENT;
  if (dtype == kFp8 && !scales) return LL_MOE_INVALID_ARGUMENT;
  if (!aligned(payload, 16) || !aligned(src_tokens, 4) || !aligned(counts, 4) ||
      !aligned(status, 4) || (dtype == kFp8 && !aligned(scales, 4)))
    return LL_MOE_INVALID_ARGUMENT;
  const uint64_t row_bytes = dtype == kBf16 ? 2 * (uint64_t)hidden : (uint64_t)hidden;
  // the outputs are written while the layout is read: no overlap
  if (overlaps(layout, L.total, payload, slots * row_bytes) ||
      overlaps(layout, L.total, src_tokens, slots * 4) ||
      overlaps(layout, L.total, counts, (uint64_t)num_experts * 4) ||
      (dtype == kFp8 && overlaps(layout, L.total, scales, slots * (hidden / 128) * 4)))
    return LL_MOE_INVALID_ARGUMENT;

  uint8_t* base = static_cast<uint8_t*>(layout);
  UnpackParams p;
  p.sig = reinterpret_cast<const unsigned long long*>(base + L.sig_off(parity));
  p.sig_other = reinterpret_cast<unsigned long long*>(base + L.sig_off(parity ^ 1));
  p.recv = base + L.recv_off(parity);
  p.payload = static_cast<uint8_t*>(payload);
  p.scales = scales;
  p.src = src_tokens;
  p.counts = counts;
  p.status = status;
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.fp8 = dtype == kFp8;
  p.msg_bytes = (uint32_t)L.dispatch_msg;
  p.row_bytes = (uint32_t)row_bytes;
  p.expected = expected;
  p.max_spins = max_spins;
  p.wide = (uint64_t)expected * L.dispatch_msg >= kStreamRowsBytes;
  const int grid = p.wide ? kUnpackWideBlocks : kUnpackBlocks;
  const int blocks = slots < grid ? (int)slots : grid;
  return from_hip(launch_dispatch_recv(p, blocks, stream));
}

extern "C" int ll_moe_clean_signals(void* layout, int max_tokens, int hidden, int num_experts,
                                    int dtype, int parity, hipStream_t stream) {
  Layout L;
  if (parity != 0 && parity != 1) return LL_MOE_INVALID_ARGUMENT;
  if (!make_layout(max_tokens, hidden, num_experts, dtype, &L)) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !aligned(layout, 16)) return LL_MOE_INVALID_ARGUMENT;
  auto* sig = reinterpret_cast<unsigned long long*>(static_cast<uint8_t*>(layout) + L.sig_off(parity));
  return from_hip(launch_clean(sig, num_experts, stream));
}

extern "C" int ll_moe_diag_e4m3(const float* in, uint8_t* out, size_t n, hipStream_t stream) {
  if (n == 0) return LL_MOE_SUCCESS;
  if (!in || !out || !aligned(in, 4)) return LL_MOE_INVALID_ARGUMENT;
  return from_hip(launch_e4m3_probe(in, out, (uint64_t)n, false, stream));
}

extern "C" int ll_moe_diag_e4m3_in_range(const float* in, uint8_t* out, size_t n,
                                         hipStream_t stream) {
  if (n == 0) return LL_MOE_SUCCESS;
  if (!in || !out || !aligned(in, 4)) return LL_MOE_INVALID_ARGUMENT;
  return from_hip(launch_e4m3_probe(in, out, (uint64_t)n, true, stream));
}

extern "C" const char* ll_moe_status_string(int status) {
  switch (status) {
    case LL_MOE_SUCCESS: return "LL_MOE_SUCCESS";
    case LL_MOE_HIP_ERROR: return "LL_MOE_HIP_ERROR";
    case LL_MOE_INTERNAL_ERROR: return "LL_MOE_INTERNAL_ERROR";
    case LL_MOE_INVALID_ARGUMENT: return "LL_MOE_INVALID_ARGUMENT";
    case LL_MOE_INVALID_USAGE: return "LL_MOE_INVALID_USAGE";
    default: return "LL_MOE_UNKNOWN_STATUS";
  }
}
