// Host-side layout arithmetic of the two-set LL MoE buffer.
//
// rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, LLMoEBufferLayout constructor:
// message sizes, send / receive / signal buffer sizes (each send and receive
// size a multiple of sizeof(int)), and the pointer table of the two sets.
// The fp8 dispatch message carries the e4m3 codes and one fp32 scale per 128
// codes; the combine message is always bf16.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace llmoe {

enum : int { kBf16 = 0, kFp8 = 1 };
constexpr int kFp8Block = 128;
constexpr int kMaxTopk = 16;
constexpr uint64_t kMaxMessageBytes = 45056;

struct Layout {
  uint64_t dispatch_msg;  // md
  uint64_t combine_msg;   // mc
  uint64_t send;          // bytes of one send buffer
  uint64_t recv;          // bytes of one receive buffer
  uint64_t sig;           // bytes of one signal array
  uint64_t total;
  uint64_t send_off(int q) const { return send * (uint64_t)q; }
  uint64_t recv_off(int q) const { return 2 * send + recv * (uint64_t)q; }
  uint64_t sig_off(int q) const { return 2 * send + 2 * recv + sig * (uint64_t)q; }
};

inline bool mul_ok(uint64_t a, uint64_t b, uint64_t* r) {
  return !__builtin_mul_overflow(a, b, r);
}
inline bool add_ok(uint64_t a, uint64_t b, uint64_t* r) {
  return !__builtin_add_overflow(a, b, r);
}

// Returns false for arguments the layout cannot describe.
inline bool make_layout(int max_tokens, int hidden, int num_experts, int dtype, Layout* L) {
  if (max_tokens < 1 || hidden < 1 || num_experts < 1) return false;
  const uint64_t n = (uint64_t)max_tokens, h = (uint64_t)hidden, e = (uint64_t)num_experts;
  uint64_t md;
  if (dtype == kBf16) {
    md = 4 + 2 * h;
  } else if (dtype == kFp8) {
    if (h % kFp8Block) return false;
    md = 4 + h + 4 * (h / kFp8Block);
  } else {
    return false;
  }
  const uint64_t mc = 4 + 2 * h;
  uint64_t en, ds, cs, dr, cr;
  if (!mul_ok(e, n, &en) || !mul_ok(n, md, &ds) || !mul_ok(en, mc, &cs) ||
      !mul_ok(en, md, &dr) || !mul_ok(en, mc, &cr))
    return false;
  const uint64_t send = ds > cs ? ds : cs;
  const uint64_t recv = dr > cr ? dr : cr;
  if (send % 4 || recv % 4) return false;
  const uint64_t sig = 8 * e;
  uint64_t t1, t2;
  if (!add_ok(send, recv, &t1) || !add_ok(t1, sig, &t2) || !mul_ok(t2, 2, &t1)) return false;
  L->dispatch_msg = md;
  L->combine_msg = mc;
  L->send = send;
  L->recv = recv;
  L->sig = sig;
  L->total = t1;
  return true;
}

}  // namespace llmoe
