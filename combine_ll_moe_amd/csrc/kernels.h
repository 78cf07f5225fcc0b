// Launchers of the gfx950 kernels; called by the C ABI in api.hip after it
// has validated the arguments. Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmoe {

struct DispatchParams {
  uint8_t* send;                   // send buffer of set q
  uint8_t* recv;                   // receive buffer of set q
  unsigned long long* sig;         // signal words of set q (accumulated)
  unsigned long long* sig_other;   // signal words of set 1-q (zeroed)
  const uint4* x;                  // bf16 [num_tokens, hidden] as 16-byte chunks
  const int32_t* idx;              // int32 [num_tokens, topk]
  int num_tokens;
  int max_tokens;
  int hidden;
  int num_experts;
  int topk;
  int tile;                        // consecutive tokens per workgroup
  int groups;                      // workgroups per tile (each takes every groups-th row)
  int group_rows;                  // LDS path: rows by whole workgroups (else by wavefronts)
  uint32_t msg_bytes;              // md
  uint32_t msg_stride;             // LDS path: bytes of one message buffer (one per tile token)
  int line_align;                  // 64 MiB of rows or more: the LDS path, whole-line stores
  int vec_idx;                     // routing table readable 4 entries per load (register path)
  int wide_idx;                    // the same, and read so on the LDS path (large tables)
};

struct CombineParams {
  unsigned long long* sig_other;   // signal words of set 1-q (zeroed)
  const uint4* y;                  // bf16 [num_experts * max_tokens, hidden] as 16-byte chunks
  const int32_t* idx;              // int32 [num_tokens, topk]
  const float* w;                  // fp32 [num_tokens, topk]
  float4* out;                     // fp32 [num_tokens, hidden]
  int num_tokens;
  int max_tokens;
  int hidden;
  int num_experts;
  int topk;
  int tile;                        // consecutive tokens per workgroup
  int slices;                      // workgroups per tile, each a contiguous run of columns
  int block;                       // threads per workgroup (one 16-byte column chunk each)
  int stream_rows;                 // read the expert rows with non-temporal loads
  int vec_idx;                     // routing table readable 4 entries per load
};

struct SendParams {                // two-phase combine, expert side
  unsigned long long* sig;         // signal words of set q (counts; flags in the high halves)
  unsigned long long* sig_other;   // signal words of set 1-q (zeroed)
  const uint8_t* recv;             // receive buffer of set q (dispatch messages)
  uint8_t* stage;                  // combine send buffer of set q (= its send buffer)
  const uint4* y;                  // bf16 [num_experts * max_tokens, hidden] as 16-byte chunks
  int max_tokens;
  int hidden;
  int num_experts;
  uint32_t msg_bytes;              // md: dispatch message bytes
  uint32_t comb_bytes;             // mc: combine message bytes
  int nbuf;                        // LDS message buffers (2: double-buffered)
};

struct RecvParams {                // two-phase combine, token side
  const unsigned long long* sig;   // signal words of set q
  unsigned long long* sig_other;   // signal words of set 1-q (zeroed)
  const uint8_t* stage;            // combine send buffer of set q
  const int32_t* idx;              // int32 [num_tokens, topk]
  const float* w;                  // fp32 [num_tokens, topk]
  float4* out;                     // fp32 [num_tokens, hidden]
  int32_t* status;                 // zeroed by the caller: ready, or a refusal
  int num_tokens;
  int max_tokens;
  int hidden;
  int num_experts;
  int topk;
  int tile;                        // consecutive tokens per workgroup
  int slices;                      // workgroups per tile, each a contiguous run of columns
  int block;                       // threads per workgroup (one 16-byte column chunk each)
  uint32_t comb_bytes;             // mc
  int max_spins;                   // polls of one flag before its wait gives up
  int stream_rows;                 // read the staging rows with non-temporal loads
};

struct UnpackParams {              // expert side of the dispatch
  const unsigned long long* sig;   // signal words of set q (counts in the low halves)
  unsigned long long* sig_other;   // signal words of set 1-q (zeroed)
  const uint8_t* recv;             // receive buffer of set q
  uint8_t* payload;                // [num_experts * max_tokens, row_bytes]
  float* scales;                   // fp8: [num_experts * max_tokens, hidden / 128]
  int32_t* src;                    // [num_experts * max_tokens] source tokens
  int32_t* counts;                 // [num_experts]
  int32_t* status;                 // zeroed by the caller: ready, or a refusal
  int max_tokens;
  int hidden;
  int num_experts;
  int fp8;                         // payload = hidden e4m3 codes, then hidden/128 scales
  uint32_t msg_bytes;              // md
  uint32_t row_bytes;              // payload bytes of one unpacked row
  int expected;                    // messages the step routes
  int max_spins;                   // polls of the counts before the wait gives up
  int wide;                        // 64 MiB of messages or more: more loads in flight per lane
};

// The two-phase combine's expert side keeps every expert's count in LDS.
constexpr int kSendMaxExperts = 4096;
constexpr int kSendBlock = 256;
// The two-phase combine's token side: at most this many workgroups (two per
// CU), looping over its work items.
constexpr int kRecvBlocks = 512;
// Refusal codes: a flag wait of ll_moe_combine_recv ran out; the count wait
// of ll_moe_dispatch_recv ran out.
constexpr int32_t kRefusalFlagWait = 1;
constexpr int32_t kRefusalCountWait = 2;
// Status of ll_moe_dispatch_recv and ll_moe_combine_recv: the wait ended
// well (the counts added up; every flag came up); and, beside it, the wait
// found the set incomplete at its first look (the call started before the
// work it waits for had finished).
constexpr int32_t kStatusReady = 0x100;
constexpr int32_t kStatusWaited = 0x200;

// LDS placement of a message: it starts at this offset of its buffer, so
// that the payload (message byte 4) is 16-byte aligned; a buffer is
// kMsgLdsOffset + md rounded up to 16 bytes.
constexpr int kMsgLdsOffset = 12;
constexpr int kDispatchBlock = 256;
constexpr int kXcds = 8;  // XCDs of an MI355X; workgroups are dealt to them round-robin

// Buffer-store cache policy with the device-scope coherence bit (sc1): the
// store writes through the XCD's L2. Raw-buffer descriptor word 3 for gfx9.
constexpr int kCachePolicySc1 = 16;
constexpr int kCachePolicyNt = 2;  // non-temporal (streaming)
constexpr int kBufferWord3 = 0x00020000;
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0)
// Combine workgroups: at most kCombineBlock threads (kCombineWideBlock for
// gathers of kStreamRowsBytes or more), kCombineMaxBlock in any case.
constexpr int kCombineBlock = 256;
constexpr int kCombineWideBlock = 448;
constexpr int kCombineMaxBlock = 512;

// Launch shapes shared by the combine and the gather probe. A workgroup
// takes a tile of consecutive tokens and one run of columns; tiles grow
// (sharing one routing prologue among more tokens) once there are enough
// workgroups to give each of the 256 CUs about two.
constexpr int kTargetBlocks = 512;
constexpr int kMaxTileTokens = 2;
constexpr int kTileEntryLimit = 64;  // tokens per tile * topk: one wavefront's lanes
// Row gathers (and dispatches) of this many bytes or more mostly miss the
// caches and take the streaming forms.
constexpr uint64_t kStreamRowsBytes = 64ull << 20;

inline int tile_for(int num_tokens, int per_token_blocks, int topk, int target = kTargetBlocks) {
  int tile = (int)(((int64_t)num_tokens * per_token_blocks) / target);
  if (tile > kMaxTileTokens) tile = kMaxTileTokens;
  if (tile > kTileEntryLimit / topk) tile = kTileEntryLimit / topk;
  return tile < 1 ? 1 : tile;
}
// The combine's launch shape: a workgroup of `block` threads (8 columns
// each) takes a tile of `tile` tokens and one of `slices` equal runs of
// columns that cover a row. Equal runs measured faster than runs of 256
// threads with a short last one (a 7168-column row in runs of 256, 256,
// 256 and 128 threads: 128 tokens 5.13 us, 1024 tokens 29.8; in four runs
// of 224: 5.04 and 29.1), although the gather alone, rows handed in,
// takes the same time in both shapes (1024 tokens: 27.9 us), and dealing
// the short runs evenly to the XCDs made the combine slower (5.95, 30.0).
// Large gathers take longer runs, fewer workgroups and so fewer routing
// prologues: two runs of 448 threads, 1024 tokens of 7168 columns in 29.0
// us. A block is a multiple of 32 threads and at least one wavefront (the
// routing prologue holds a tile's entries in wavefront 0's lanes).
struct CombineShape {
  int slices, tile, block;
};
inline CombineShape combine_shape(int num_tokens, int hidden, int topk, bool stream_rows) {
  CombineShape s;
  const int chunks = hidden / 8;
  const int most = stream_rows ? kCombineWideBlock : kCombineBlock;
  s.slices = (chunks + most - 1) / most;
  const int even = (chunks + s.slices - 1) / s.slices;
  s.block = (even + 31) / 32 * 32;
  if (s.block < 64) s.block = 64;
  s.tile = tile_for(num_tokens, s.slices, topk);
  return s;
}

hipError_t launch_dispatch(const DispatchParams& p, int dtype, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_combine_send(const SendParams& p, int blocks, hipStream_t stream);
hipError_t launch_combine_recv(const RecvParams& p, hipStream_t stream);
hipError_t launch_dispatch_recv(const UnpackParams& p, int blocks, hipStream_t stream);
hipError_t launch_clean(unsigned long long* sig, int num_experts, hipStream_t stream);
hipError_t launch_e4m3_probe(const float* in, uint8_t* out, uint64_t n, bool in_range,
                             hipStream_t stream);

}  // namespace llmoe
