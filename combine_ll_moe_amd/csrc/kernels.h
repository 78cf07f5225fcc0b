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
  int groups;                      // workgroups per token (each takes every groups-th message)
  uint32_t msg_bytes;              // md
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
  int slices;                      // workgroups per token, each a contiguous run of columns
};

hipError_t launch_dispatch(const DispatchParams& p, int dtype, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_clean(unsigned long long* sig, int num_experts, hipStream_t stream);
hipError_t launch_e4m3_probe(const float* in, uint8_t* out, uint64_t n, hipStream_t stream);

}  // namespace llmoe
