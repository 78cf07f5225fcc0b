/*
 * CPU oracle for the low-latency MoE dispatch + combine step.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
 * CPU-baseline leg load the library built from this file. The GPU library
 * never includes, links or calls it, and this file includes nothing of the
 * GPU library: constants, sizes and helpers are written out again here.
 *
 * Everything is a plain loop in the order the definition states it, so that
 * a reader can check it against the sources by eye. Sources, by page and
 * construct:
 *   [rocSHMEM LL_MoE_Buffers.hpp]  struct LLMoEBuffer (buffer roles and
 *       shapes), the LLMoEBufferLayout<T> constructor (message sizes, send /
 *       receive / signal buffer sizes, the two-set pointer table),
 *       clean_meta(), get_rdma_size_hint<T>().
 *   [mscclpp.h]  the put / signal / wait contract in the comment above
 *       struct mscclppDevConn: data first, then the signal; the receiver
 *       reads only after it has seen the signal.
 *   [memra-engine tp_ar.rs]  memra_tp_ar_1stage: operands are combined in a
 *       fixed order so that every caller forms the same expression.
 * Where the pages leave a step open, the reading taken is stated at the
 * function that takes it.
 *
 * Floating point: the combine accumulates in fp32 with fmaf in ascending k,
 * which is the precision the method fixes; the fp8 quantizer is fp32
 * throughout (its scales are fp32 values stored in the message).
 * Build with -ffp-contract=off so that no expression is fused behind fmaf's
 * back.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(__BYTE_ORDER__) || __BYTE_ORDER__ != __ORDER_LITTLE_ENDIAN__
#error "the oracle writes little-endian words with memcpy"
#endif

enum { OR_BF16 = 0, OR_FP8_E4M3 = 1 };
enum { OR_FP8_BLOCK = 128 };

/* ---------------------------------------------------------------------------
 * Message sizes.
 * [rocSHMEM LL_MoE_Buffers.hpp, LLMoEBufferLayout constructor, "Message
 * sizes"]: a message is one int (the source token index) followed by hidden
 * payload elements of type T, with no padding.
 * Reading: the dispatch payload may be fp8 e4m3, in which case each message
 * also carries one fp32 scale per 128 payload elements, appended after the
 * payload; the combine message always carries bf16 (the combine input is
 * bf16), so its size does not depend on the dispatch dtype.
 * ------------------------------------------------------------------------- */
int oracle_message_bytes(int hidden, int dtype, uint64_t* dispatch_bytes,
                         uint64_t* combine_bytes) {
  if (hidden <= 0) return -1;
  uint64_t h = (uint64_t)hidden;
  uint64_t md;
  if (dtype == OR_BF16) {
    md = 4 + h * 2;
  } else if (dtype == OR_FP8_E4M3) {
    if (h % OR_FP8_BLOCK != 0) return -1;
    md = 4 + h * 1 + 4 * (h / OR_FP8_BLOCK);
  } else {
    return -1;
  }
  *dispatch_bytes = md;
  *combine_bytes = 4 + h * 2;
  return 0;
}

/* ---------------------------------------------------------------------------
 * Layout: [rocSHMEM LL_MoE_Buffers.hpp, LLMoEBufferLayout constructor].
 *   send bytes  = max(tokens * dispatch msg, experts * tokens * combine msg)
 *   recv bytes  = max(experts * tokens * dispatch msg,
 *                     experts * tokens * combine msg)
 *   both must be a multiple of sizeof(int) (the constructor's ASSERTs)
 *   signal bytes = experts * sizeof(int64_t)
 *   total = 2 * send + 2 * recv + 2 * signal
 * Pointer table for set i (i = 0, 1): send at i * send, recv at 2 * send +
 * i * recv, signal at 2 * send + 2 * recv + i * signal. Within one set the
 * combine pointers equal the dispatch pointers.
 * out[0] = total, out[1+i] = send offset, out[3+i] = recv offset,
 * out[5+i] = signal offset.
 * ------------------------------------------------------------------------- */
int oracle_layout(int max_tokens, int hidden, int num_experts, int dtype,
                  uint64_t out[7]) {
  uint64_t md, mc;
  if (max_tokens <= 0 || num_experts <= 0) return -1;
  if (oracle_message_bytes(hidden, dtype, &md, &mc) != 0) return -1;
  uint64_t n = (uint64_t)max_tokens, e = (uint64_t)num_experts;

  uint64_t dispatch_send = n * md;
  uint64_t combine_send = e * n * mc;
  uint64_t send = dispatch_send > combine_send ? dispatch_send : combine_send;
  if (send % 4 != 0) return -1;

  uint64_t dispatch_recv = e * n * md;
  uint64_t combine_recv = e * n * mc;
  uint64_t recv = dispatch_recv > combine_recv ? dispatch_recv : combine_recv;
  if (recv % 4 != 0) return -1;

  uint64_t sig = e * 8;

  out[0] = send * 2 + recv * 2 + sig * 2;
  for (int i = 0; i < 2; ++i) {
    out[1 + i] = send * (uint64_t)i;
    out[3 + i] = send * 2 + recv * (uint64_t)i;
    out[5 + i] = send * 2 + recv * 2 + sig * (uint64_t)i;
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * fp32 -> OCP fp8 e4m3 ("e4m3fn": bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448, smallest subnormal 2^-9).
 * Rounding to nearest, ties to even; finite values beyond 448 and the
 * infinities saturate to +-448; every NaN maps to 0x7F.
 * The pages give no quantizer: this is the reading taken (round to nearest
 * even, saturate, NaN sign dropped).
 * Written as: find the spacing of the e4m3 grid around |v|, count spacings
 * with round-half-even, then write exponent and mantissa fields.
 * ------------------------------------------------------------------------- */
uint8_t oracle_e4m3(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;

  double min_normal = ldexp(1.0, -6);
  double spacing;
  if (a < min_normal) {
    spacing = ldexp(1.0, -9); /* subnormal grid */
  } else {
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): binade [2^(ex-1), 2^ex) */
    spacing = ldexp(1.0, ex - 1 - 3);
  }
  double n = nearbyint(a / spacing); /* a / spacing is exact; RNE */
  double r = n * spacing;            /* the chosen grid value */

  uint8_t code;
  if (r < min_normal) {
    code = (uint8_t)n; /* subnormal: mantissa field counts 2^-9 steps */
  } else {
    int ex;
    frexp(r, &ex);
    int exp_field = (ex - 1) + 7;
    int mant_field = (int)(r / ldexp(1.0, ex - 1 - 3)) - 8;
    code = (uint8_t)((exp_field << 3) | mant_field);
  }
  return sign | code;
}

void oracle_e4m3_many(const float* in, uint8_t* out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = oracle_e4m3(in[i]);
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ---------------------------------------------------------------------------
 * One dispatch message for token t.
 * Bytes [0, 4): the source token index t as a little-endian int32, first,
 * as in [rocSHMEM LL_MoE_Buffers.hpp, "Message sizes"] (sizeof(int) before
 * the payload).
 * bf16: bytes [4, 4 + 2h) are the bits of x[t], unchanged.
 * fp8 (reading): for each block b of 128 elements,
 *   amax  = largest |x| in the block (NaN elements do not take part),
 *   inv   = 448 / amax and scale = amax / 448, each one correctly rounded
 *           fp32 division; both are 0 when amax is 0,
 *   q[c]  = e4m3(x[c] * inv) with one fp32 rounding of the product;
 * bytes [4, 4 + h) hold q and bytes [4 + h, md) the scales, in block order,
 * as fp32 little-endian.
 * ------------------------------------------------------------------------- */
int oracle_encode_message(int hidden, int dtype, int t, const uint16_t* xrow,
                          uint8_t* msg) {
  uint64_t md, mc;
  if (oracle_message_bytes(hidden, dtype, &md, &mc) != 0) return -1;
  int32_t header = t;
  memcpy(msg, &header, 4);
  if (dtype == OR_BF16) {
    for (int c = 0; c < hidden; ++c) {
      uint16_t b = xrow[c];
      memcpy(msg + 4 + 2 * (uint64_t)c, &b, 2);
    }
    return 0;
  }
  int nblocks = hidden / OR_FP8_BLOCK;
  uint8_t* q = msg + 4;
  uint8_t* scales = msg + 4 + hidden;
  for (int b = 0; b < nblocks; ++b) {
    float amax = 0.0f;
    for (int c = 0; c < OR_FP8_BLOCK; ++c) {
      float a = fabsf(bf16_to_f32(xrow[b * OR_FP8_BLOCK + c]));
      if (a > amax) amax = a;
    }
    float inv = 0.0f, scale = 0.0f;
    if (amax > 0.0f) {
      inv = 448.0f / amax;
      scale = amax / 448.0f;
    }
    for (int c = 0; c < OR_FP8_BLOCK; ++c) {
      float p = bf16_to_f32(xrow[b * OR_FP8_BLOCK + c]) * inv;
      q[b * OR_FP8_BLOCK + c] = oracle_e4m3(p);
    }
    memcpy(scales + 4 * (uint64_t)b, &scale, 4);
  }
  return 0;
}

int oracle_encode_messages(int num_tokens, int hidden, int dtype,
                           const uint16_t* x, uint8_t* msgs) {
  uint64_t md, mc;
  if (oracle_message_bytes(hidden, dtype, &md, &mc) != 0) return -1;
  for (int t = 0; t < num_tokens; ++t)
    if (oracle_encode_message(hidden, dtype, t, x + (uint64_t)t * hidden,
                              msgs + (uint64_t)t * md) != 0)
      return -1;
  return 0;
}

/* ---------------------------------------------------------------------------
 * Routing: per-expert counts and the receive slot of every (t, k).
 * The receive buffer holds num_experts * num_tokens messages
 * [rocSHMEM LL_MoE_Buffers.hpp, struct LLMoEBuffer, dispatch recv buffer
 * shape], read here as experts-major: expert e owns rows
 * [e * max_tokens, (e + 1) * max_tokens).
 * Readings:
 *   - slots are handed out in ascending token order, and for one token in
 *     ascending k: one running counter per expert, walked over (t, k);
 *   - an entry outside [0, num_experts) is masked: no slot, not counted;
 *   - an entry that would get a slot >= max_tokens (possible only when a
 *     token repeats an expert) is dropped the same way, so that no write
 *     leaves the expert's rows.
 * slot[t * K + k] = -1 marks a masked or dropped entry.
 * ------------------------------------------------------------------------- */
int oracle_route(int num_tokens, int topk, int num_experts, int max_tokens,
                 const int32_t* idx, int32_t* slot, int64_t* cnt) {
  if (num_tokens < 0 || topk <= 0 || num_experts <= 0 || max_tokens <= 0)
    return -1;
  for (int e = 0; e < num_experts; ++e) cnt[e] = 0;
  for (int t = 0; t < num_tokens; ++t) {
    for (int k = 0; k < topk; ++k) {
      int32_t e = idx[(uint64_t)t * topk + k];
      int32_t s = -1;
      if (e >= 0 && e < num_experts && cnt[e] < max_tokens) {
        s = (int32_t)cnt[e];
        cnt[e] += 1;
      }
      slot[(uint64_t)t * topk + k] = s;
    }
  }
  return 0;
}

static int check_call(int max_tokens, int num_tokens, int hidden,
                      int num_experts, int topk, int dtype, int parity,
                      uint64_t lay[7]) {
  if (parity != 0 && parity != 1) return -1;
  if (num_tokens < 0 || num_tokens > max_tokens) return -1;
  if (topk < 1 || topk > num_experts) return -1;
  return oracle_layout(max_tokens, hidden, num_experts, dtype, lay);
}

static void put_i64(uint8_t* p, int64_t v) { memcpy(p, &v, 8); }
static int64_t get_i64(const uint8_t* p) {
  int64_t v;
  memcpy(&v, p, 8);
  return v;
}

/* ---------------------------------------------------------------------------
 * Dispatch with parity q on a host image of the whole layout.
 *  1. the other set's signal words are zeroed (the clean of the next-parity
 *     buffer, [rocSHMEM LL_MoE_Buffers.hpp, clean_meta()]: one clean covers
 *     the dispatch count words and the combine flag words, which are the
 *     same address);
 *  2. message t is written to send row t of set q ([LLMoEBuffer] dispatch
 *     send buffer, one row per token);
 *  3. for every routed (t, k) the same message is written to receive row
 *     e * max_tokens + slot(t, k) of set q;
 *  4. each expert's signal word of set q is increased by the number of
 *     messages it received (the dispatch recv count buffer, int64 per
 *     expert). The word counts arrivals since its last clean; the GPU side
 *     publishes it only after the messages, as in [mscclpp.h] (signal after
 *     put), which a value check cannot see.
 * No other byte of the image changes.
 * ------------------------------------------------------------------------- */
int oracle_dispatch(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                    int num_experts, int topk, int dtype, int parity,
                    const uint16_t* x, const int32_t* idx) {
  uint64_t lay[7], md, mc;
  if (check_call(max_tokens, num_tokens, hidden, num_experts, topk, dtype,
                 parity, lay) != 0)
    return -1;
  oracle_message_bytes(hidden, dtype, &md, &mc);
  uint8_t* send = image + lay[1 + parity];
  uint8_t* recv = image + lay[3 + parity];
  uint8_t* sig = image + lay[5 + parity];
  uint8_t* sig_other = image + lay[5 + (parity ^ 1)];

  for (int e = 0; e < num_experts; ++e) put_i64(sig_other + 8 * (uint64_t)e, 0);

  uint64_t nk = (uint64_t)num_tokens * topk;
  int32_t* slot = malloc((nk ? nk : 1) * sizeof(int32_t));
  int64_t* cnt = malloc((uint64_t)num_experts * sizeof(int64_t));
  uint8_t* msg = malloc(md);
  if (!slot || !cnt || !msg) {
    free(slot);
    free(cnt);
    free(msg);
    return -1;
  }
  oracle_route(num_tokens, topk, num_experts, max_tokens, idx, slot, cnt);

  for (int t = 0; t < num_tokens; ++t) {
    oracle_encode_message(hidden, dtype, t, x + (uint64_t)t * hidden, msg);
    memcpy(send + (uint64_t)t * md, msg, md);
    for (int k = 0; k < topk; ++k) {
      int32_t s = slot[(uint64_t)t * topk + k];
      if (s < 0) continue;
      uint64_t e = (uint64_t)idx[(uint64_t)t * topk + k];
      memcpy(recv + (e * (uint64_t)max_tokens + (uint64_t)s) * md, msg, md);
    }
  }
  for (int e = 0; e < num_experts; ++e) {
    uint8_t* w = sig + 8 * (uint64_t)e;
    put_i64(w, get_i64(w) + cnt[e]);
  }
  free(slot);
  free(cnt);
  free(msg);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Combine with parity q.
 * expert_out is bf16 [num_experts * max_tokens, hidden] in receive-slot
 * order: row e * max_tokens + j is expert e's output for the j-th message it
 * received. For every token t and column c:
 *     acc = +0.0f;  for k = 0 .. K-1 (routed entries only):
 *         acc = fmaf(w[t, k], f32(expert_out[e * max_tokens + slot(t, k), c]), acc)
 *     out[t, c] = acc
 * The top-k weighted sum in fp32, operands taken in one fixed order (as the
 * one-shot all-reduce of [memra-engine tp_ar.rs, memra_tp_ar_1stage] fixes
 * its operand order so every caller forms the same expression). slot(t, k)
 * is the routing function above; the image's data buffers are not read.
 * Then the other set's signal words are zeroed, as every launch of parity q
 * does. No other byte of the image changes.
 * ------------------------------------------------------------------------- */
int oracle_combine(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                   int num_experts, int topk, int dtype, int parity,
                   const uint16_t* expert_out, const int32_t* idx,
                   const float* weights, float* out) {
  uint64_t lay[7];
  if (check_call(max_tokens, num_tokens, hidden, num_experts, topk, dtype,
                 parity, lay) != 0)
    return -1;
  uint64_t nk = (uint64_t)num_tokens * topk;
  int32_t* slot = malloc((nk ? nk : 1) * sizeof(int32_t));
  int64_t* cnt = malloc((uint64_t)num_experts * sizeof(int64_t));
  if (!slot || !cnt) {
    free(slot);
    free(cnt);
    return -1;
  }
  oracle_route(num_tokens, topk, num_experts, max_tokens, idx, slot, cnt);

  for (int t = 0; t < num_tokens; ++t) {
    float* o = out + (uint64_t)t * hidden;
    for (int c = 0; c < hidden; ++c) o[c] = 0.0f;
    for (int k = 0; k < topk; ++k) {
      int32_t s = slot[(uint64_t)t * topk + k];
      if (s < 0) continue;
      uint64_t e = (uint64_t)idx[(uint64_t)t * topk + k];
      const uint16_t* row =
          expert_out + (e * (uint64_t)max_tokens + (uint64_t)s) * hidden;
      float w = weights[(uint64_t)t * topk + k];
      for (int c = 0; c < hidden; ++c) o[c] = fmaf(w, bf16_to_f32(row[c]), o[c]);
    }
  }
  uint8_t* sig_other = image + lay[5 + (parity ^ 1)];
  for (int e = 0; e < num_experts; ++e) put_i64(sig_other + 8 * (uint64_t)e, 0);
  free(slot);
  free(cnt);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Two-phase combine with parity q: the combine as a put of the expert
 * outputs plus a flag hand-off, on a host image of the layout after
 * dispatch(q). The pages give the buffers and the put / signal / wait
 * contract, not this protocol; the readings taken:
 *  - a combine message is int32 t followed by the bf16 output row
 *    ([rocSHMEM LL_MoE_Buffers.hpp], "Message sizes", the combine message),
 *    mc = 4 + 2h bytes;
 *  - the expert side stages expert e's message for token t in set q's
 *    combine send buffer at row e * max_tokens + t. The pointer table makes
 *    that buffer the dispatch send buffer, whose rows are spent once the
 *    dispatch is done; the combine receive buffer of set q is the dispatch
 *    receive buffer, whose rows this phase still reads. On one device the
 *    receiver reads the staged rows where they are: the put is the
 *    identity;
 *  - expert e's flag is set q's signal word e (clean_meta(): the dispatch
 *    count words and the combine flag words are one array). The expert side
 *    adds the number of rows it delivered to the word's high 32 bits, after
 *    the rows ([mscclpp.h]: data first, then the signal); the receiver takes
 *    expert e's rows once the high half equals the low half, the dispatch
 *    count;
 *  - a token names an expert at most once (the staging row is per expert
 *    and token).
 * Each launch zeroes the other set's signal words, as every launch of
 * parity q does.
 * ------------------------------------------------------------------------- */

/* Expert side: for every expert e and slot j below its count (the low half
 * of signal word e), t = the header of receive row e * max_tokens + j, and
 * staging row e * max_tokens + t = message(t, expert_out row
 * e * max_tokens + j); then signal word e += count << 32. */
int oracle_combine_send(uint8_t* image, int max_tokens, int hidden, int num_experts,
                        int dtype, int parity, const uint16_t* expert_out) {
  uint64_t lay[7], md, mc;
  if (check_call(max_tokens, 0, hidden, num_experts, 1, dtype, parity, lay) != 0)
    return -1;
  oracle_message_bytes(hidden, dtype, &md, &mc);
  uint8_t* stage = image + lay[1 + parity];
  const uint8_t* recv = image + lay[3 + parity];
  uint8_t* sig = image + lay[5 + parity];
  uint8_t* sig_other = image + lay[5 + (parity ^ 1)];
  for (int e = 0; e < num_experts; ++e) put_i64(sig_other + 8 * (uint64_t)e, 0);
  for (int e = 0; e < num_experts; ++e) {
    uint8_t* w = sig + 8 * (uint64_t)e;
    int64_t word = get_i64(w);
    int64_t count = word & 0xFFFFFFFF;
    if (count > max_tokens) return -1;
    for (int64_t j = 0; j < count; ++j) {
      uint64_t src = (uint64_t)e * (uint64_t)max_tokens + (uint64_t)j;
      int32_t t;
      memcpy(&t, recv + src * md, 4);
      if (t < 0 || t >= max_tokens) return -1;
      uint8_t* dst = stage + ((uint64_t)e * (uint64_t)max_tokens + (uint64_t)t) * mc;
      memcpy(dst, &t, 4);
      memcpy(dst + 4, expert_out + src * (uint64_t)hidden, 2 * (uint64_t)hidden);
    }
    put_i64(w, word + (int64_t)((uint64_t)count << 32));
  }
  return 0;
}

/* Token side: every routed pick of token t needs expert e's flag (high half
 * of signal word e equal to its low half); then
 *     out[t, c] = fma chain in ascending k, from +0.0f, of
 *                 w[t, k] * f32(staging row e * max_tokens + t, column c).
 * Returns -2 if a needed flag is not raised (the GPU side reports that in its
 * refusal word instead of waiting forever). */
int oracle_combine_recv(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                        int num_experts, int topk, int dtype, int parity,
                        const int32_t* idx, const float* weights, float* out) {
  uint64_t lay[7], md, mc;
  if (check_call(max_tokens, num_tokens, hidden, num_experts, topk, dtype, parity, lay) != 0)
    return -1;
  oracle_message_bytes(hidden, dtype, &md, &mc);
  const uint8_t* stage = image + lay[1 + parity];
  const uint8_t* sig = image + lay[5 + parity];
  uint8_t* sig_other = image + lay[5 + (parity ^ 1)];
  for (int t = 0; t < num_tokens; ++t) {
    float* o = out + (uint64_t)t * hidden;
    for (int c = 0; c < hidden; ++c) o[c] = 0.0f;
    for (int k = 0; k < topk; ++k) {
      int32_t e = idx[(uint64_t)t * topk + k];
      if (e < 0 || e >= num_experts) continue;
      int64_t word = get_i64(sig + 8 * (uint64_t)e);
      if ((word >> 32) != (word & 0xFFFFFFFF)) return -2;
      const uint8_t* row = stage + ((uint64_t)e * (uint64_t)max_tokens + (uint64_t)t) * mc + 4;
      float w = weights[(uint64_t)t * topk + k];
      for (int c = 0; c < hidden; ++c) {
        uint16_t b;
        memcpy(&b, row + 2 * (uint64_t)c, 2);
        o[c] = fmaf(w, bf16_to_f32(b), o[c]);
      }
    }
  }
  for (int e = 0; e < num_experts; ++e) put_i64(sig_other + 8 * (uint64_t)e, 0);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Expert side of the dispatch with parity q: wait for the dispatch's
 * messages, then unpack them into the form an expert's matrix product
 * reads. The pages give the receive rows, the per-expert counts and
 * [mscclpp.h]'s rule that a receiver reads only after the signal, not this
 * step; the readings taken:
 *  - the receiver knows how many messages the step routes (`expected`) and
 *    takes set q as complete when the counts (low halves of its signal
 *    words) add up to that number. A partial count does not tell which of
 *    an expert's slots are written; the sum reaching the total does;
 *  - unpacked, receive row r = e * max_tokens + j (j below count_e) gives
 *    its payload without the header in a row of its own (bf16: the 2h bytes
 *    of x; fp8: the h codes, and the h/128 fp32 scales in a second array),
 *    its header in an int32 array, and count_e goes to an int32 array.
 *    Bytes move unchanged; rows at or past count_e are not written;
 *  - a count above max_tokens is taken as max_tokens, in the sum as in the
 *    unpacking.
 * The launch zeroes the other set's signal words first, as every launch of
 * parity q does. Returns -2 (and writes no output) when the counts do not
 * add up to `expected`: the GPU side reports that in a refusal word after
 * a bounded wait.
 * ------------------------------------------------------------------------- */
int oracle_dispatch_recv(uint8_t* image, int max_tokens, int hidden, int num_experts,
                         int dtype, int parity, int expected, uint8_t* payload,
                         float* scales, int32_t* src, int32_t* counts) {
  uint64_t lay[7], md, mc;
  if (check_call(max_tokens, 0, hidden, num_experts, 1, dtype, parity, lay) != 0)
    return -1;
  oracle_message_bytes(hidden, dtype, &md, &mc);
  const uint8_t* recv = image + lay[3 + parity];
  const uint8_t* sig = image + lay[5 + parity];
  uint8_t* sig_other = image + lay[5 + (parity ^ 1)];
  for (int e = 0; e < num_experts; ++e) put_i64(sig_other + 8 * (uint64_t)e, 0);
  int64_t total = 0;
  for (int e = 0; e < num_experts; ++e) {
    int64_t c = get_i64(sig + 8 * (uint64_t)e) & 0xFFFFFFFF;
    total += c > max_tokens ? max_tokens : c;
  }
  if (total != (int64_t)expected) return -2;
  const uint64_t row_bytes = dtype == OR_BF16 ? 2 * (uint64_t)hidden : (uint64_t)hidden;
  const uint64_t nscales = (uint64_t)hidden / OR_FP8_BLOCK;
  for (int e = 0; e < num_experts; ++e) {
    int64_t c = get_i64(sig + 8 * (uint64_t)e) & 0xFFFFFFFF;
    if (c > max_tokens) c = max_tokens;
    counts[e] = (int32_t)c;
    for (int64_t j = 0; j < c; ++j) {
      const uint64_t r = (uint64_t)e * (uint64_t)max_tokens + (uint64_t)j;
      const uint8_t* row = recv + r * md;
      memcpy(&src[r], row, 4);
      memcpy(payload + r * row_bytes, row + 4, row_bytes);
      if (dtype == OR_FP8_E4M3) memcpy(scales + r * nscales, row + 4 + hidden, 4 * nscales);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Explicit clean of set q's signal words: [rocSHMEM LL_MoE_Buffers.hpp,
 * clean_meta()] returns the signal pointer and num_sig_elems (= experts)
 * words to zero.
 * ------------------------------------------------------------------------- */
int oracle_clean(uint8_t* image, int max_tokens, int hidden, int num_experts,
                 int dtype, int parity) {
  uint64_t lay[7];
  if (parity != 0 && parity != 1) return -1;
  if (oracle_layout(max_tokens, hidden, num_experts, dtype, lay) != 0) return -1;
  uint8_t* sig = image + lay[5 + parity];
  for (int e = 0; e < num_experts; ++e) put_i64(sig + 8 * (uint64_t)e, 0);
  return 0;
}
