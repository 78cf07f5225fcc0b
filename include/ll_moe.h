/*
 * ll_moe.h — C ABI of the low-latency MoE dispatch + combine step on one
 * MI355X (gfx950). Library: libllmoe.so.
 *
 * The step, as the pages describe it:
 *   - rocSHMEM example "LL_MoE/LL_MoE_Buffers.hpp": all buffers are
 *     allocated once, sized for the worst-case decode micro-batch (file
 *     comment "Buffer sizing and allocation (DeepEP LL mode style)"); two
 *     buffer sets for double buffering (struct LLMoEBufferLayout); per set a
 *     send buffer [num_tokens, hidden+1], a receive buffer
 *     [num_experts * num_tokens, hidden+1] and one int64 signal word per
 *     expert (struct LLMoEBuffer); a message is an int followed by hidden
 *     payload elements (constructor, "Message sizes").
 *   - mscclpp "mscclpp.h", comment above struct mscclppDevConn: data is put
 *     first and signalled after; a receiver reads only after it has seen the
 *     signal.
 * Dispatch packs every token's top-k copies into per-expert receive slots
 * and publishes per-expert counts; combine gathers the expert outputs back
 * to their tokens as a top-k weighted sum in fp32.
 *
 * Conventions for every call:
 *   - Pointers are device pointers (hipMalloc or equivalent) unless stated.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronizes: a call validates its arguments, enqueues one kernel on
 *     `stream` and returns. Buffers must stay alive until the stream has
 *     run the work. Calls may be captured into a HIP graph.
 *   - Return value: an ll_moe_status_t. Argument errors are found before
 *     anything is enqueued and leave every buffer untouched. Errors in the
 *     data (expert ids) are not errors: see "routing" below.
 *   - Workloads: max_tokens >= 1, 0 <= num_tokens <= max_tokens,
 *     1 <= topk <= min(num_experts, LL_MOE_MAX_TOPK),
 *     num_experts <= LL_MOE_MAX_EXPERTS, max_tokens * topk < 2^31; bf16
 *     needs hidden % 8 == 0, fp8 needs hidden % 128 == 0; a dispatch message
 *     may not exceed LL_MOE_MAX_MESSAGE_BYTES (bf16: hidden <= 22520).
 *
 * Routing (topk_idx, int32 [num_tokens, topk], row-major):
 *   Entry (t, k) names the expert of token t's k-th pick. Expert e owns the
 *   receive rows [e * max_tokens, (e + 1) * max_tokens) of a set. Slots are
 *   handed out in ascending token order, and in ascending k within a token:
 *   slot(t, k) is the number of earlier entries (in (t, k) order) naming the
 *   same expert. An entry outside [0, num_experts) is masked (no message, no
 *   count, no combine term); so is an entry whose slot would reach
 *   max_tokens, which only a token naming one expert twice can cause.
 *
 * Parity schedule: every launch with parity q zeroes the signal words of
 * set 1-q (the clean of the next-parity buffer, struct LLMoEBuffer's
 * clean_meta() in the rocSHMEM example); dispatch(q) adds its counts to the
 * signal words of set q, which must be zero when it starts. Step s of a
 * decode loop runs dispatch(s & 1) then combine(s & 1). After allocating a
 * layout, clean both sets once (ll_moe_clean_signals with q = 0 and 1).
 * A signal word counts at most 2^32 - 1 messages between cleans (the
 * dispatch adds to its low 32 bits; one dispatch adds fewer than 2^31).
 */
#ifndef LL_MOE_H_
#define LL_MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Payload type of a dispatch message. */
typedef enum {
  LL_MOE_BF16 = 0,      /* hidden bf16 values, unchanged bits */
  LL_MOE_FP8_E4M3 = 1   /* hidden OCP e4m3 codes + hidden/128 fp32 scales */
} ll_moe_dtype_t;

/* Status codes; the numbering follows mscclpp.h's mscclppResult_t. */
typedef enum {
  LL_MOE_SUCCESS = 0,
  LL_MOE_HIP_ERROR = 1,         /* the HIP runtime refused the launch */
  LL_MOE_INTERNAL_ERROR = 3,
  LL_MOE_INVALID_ARGUMENT = 4,  /* see the conventions above */
  LL_MOE_INVALID_USAGE = 5
} ll_moe_status_t;

#define LL_MOE_MAX_TOPK 16
#define LL_MOE_MAX_MESSAGE_BYTES 45056
#define LL_MOE_MAX_EXPERTS (1 << 20)

/*
 * ll_moe_layout_bytes — bytes of one layout (both buffer sets).
 * rocSHMEM example LL_MoE_Buffers.hpp, LLMoEBufferLayout constructor and
 * get_rdma_size_hint(): with md = dispatch message bytes and mc = combine
 * message bytes,
 *   send = max(max_tokens * md, num_experts * max_tokens * mc)
 *   recv = max(num_experts * max_tokens * md, num_experts * max_tokens * mc)
 *   total = 2 * send + 2 * recv + 2 * (8 * num_experts).
 * md = 4 + 2 * hidden (bf16) or 4 + hidden + 4 * (hidden / 128) (fp8: the
 * e4m3 codes, then one fp32 scale per 128 codes); mc = 4 + 2 * hidden
 * always (the combine carries bf16). The result is the same for both
 * dtypes. Host only; enqueues nothing.
 *   out_bytes (host pointer): receives the total.
 * Errors: INVALID_ARGUMENT for sizes out of range, a send or receive size
 * that is not a multiple of 4 (the constructor's ASSERTs), or overflow.
 */
int ll_moe_layout_bytes(int max_tokens, int hidden, int num_experts, int dtype,
                        size_t* out_bytes);

/*
 * ll_moe_layout_offsets — byte offsets of set `parity` inside a layout:
 * the pointer table of the LLMoEBufferLayout constructor ("Assign
 * pointers"): send at parity * send, receive at 2 * send + parity * recv,
 * signal words at 2 * send + 2 * recv + parity * 8 * num_experts. Within a
 * set the combine buffers alias the dispatch buffers. Host only.
 *   send_off, recv_off, sig_off (host pointers): receive the offsets.
 *   msg_bytes (host pointer, may be NULL): receives md.
 */
int ll_moe_layout_offsets(int max_tokens, int hidden, int num_experts, int dtype,
                          int parity, size_t* send_off, size_t* recv_off,
                          size_t* sig_off, size_t* msg_bytes);

/*
 * ll_moe_dispatch — pack every token's messages into set `parity`.
 * Defined by the rocSHMEM example "LL_MoE/LL_MoE_Buffers.hpp": struct
 * LLMoEBuffer (the dispatch send buffer [num_tokens, hidden+1], the receive
 * buffer [num_experts * num_tokens, hidden+1] in per-expert slots and the
 * int64 count per expert) and the LLMoEBufferLayout constructor ("Message
 * sizes": an int header, then hidden payload elements); the count is raised
 * after the messages it counts as mscclpp.h's put-then-signal contract
 * (comment above struct mscclppDevConn) orders a signal after its data. The
 * pages do not say which slot a message takes; here slots go in ascending
 * (token, pick) order, and the fp8 payload's quantizer (below) is likewise
 * a reading of the pages, which give none.
 *   layout:   device, ll_moe_layout_bytes bytes, 16-byte aligned.
 *   x:        device, bf16 [num_tokens, hidden] row-major, 16-byte aligned.
 *   topk_idx: device, int32 [num_tokens, topk], 4-byte aligned.
 * Writes, for set q = parity:
 *   send row t (t < num_tokens), at send_q + t * md: message(t);
 *   receive row e * max_tokens + slot(t, k), at recv_q + row * md, for every
 *     routed (t, k): message(t);
 *   signal word e of set q: increased by the number of messages expert e
 *     received, published with device-scope release semantics after those
 *     messages (a reader that acquires the word sees them);
 *   signal words of set 1-q: zeroed.
 * message(t) = int32 t (little-endian), then for bf16 the bits of x[t],
 * for fp8 per 128-element block: amax = largest |x| (NaN ignored),
 * codes e4m3(x * (448 / amax)) rounded to nearest even and saturated to
 * +-448 (NaN -> 0x7F), then the hidden/128 scales amax / 448 as fp32
 * (amax = 0 gives scale 0 and zero codes).
 * No other byte of the layout is written. Enqueued on `stream`.
 */
int ll_moe_dispatch(void* layout, int max_tokens, int num_tokens, int hidden,
                    int num_experts, int topk, int dtype, int parity,
                    const void* x, const int32_t* topk_idx, hipStream_t stream);

/*
 * ll_moe_combine — top-k weighted sum of the expert outputs per token.
 * The rocSHMEM example's combine buffers (struct LLMoEBuffer: combine send
 * and receive buffers and a flag per expert) carry the expert outputs back
 * to their tokens; on one GPU the put and the fold collapse into one
 * gather, as memra-engine "src/tp_ar.rs" replaces its push-then-fold
 * all-reduce (memra_tp_ar_push, memra_tp_ar_fold) with a one-shot
 * memra_tp_ar_1stage that reads every input in one global order, so that
 * the result is the same bits on every call. The weighted sum is taken as
 * fmaf in ascending pick order from +0.0f (the pages fix no arithmetic; the
 * two-phase form with the flag hand-off is ll_moe_combine_send / _recv).
 *   layout:       device, as for dispatch (only the signal words of set
 *                 1-parity are written: zeroed).
 *   expert_out:   device, bf16 [num_experts * max_tokens, hidden], 16-byte
 *                 aligned, in receive-slot order: row e * max_tokens + j is
 *                 expert e's output for the j-th message it received.
 *                 Only rows of routed (t, k) contribute. Every load is
 *                 unconditional: a pick that is not routed reads a routed
 *                 pick's row of its token instead, or row 0 when none is
 *                 routed, and that value is never used. No row outside
 *                 the buffer is read.
 *   topk_idx:     device, int32 [num_tokens, topk] (the dispatch routing).
 *   topk_weights: device, fp32 [num_tokens, topk].
 *   out:          device, fp32 [num_tokens, hidden], 16-byte aligned; may
 *                 not overlap expert_out.
 * out[t, c] = fma chain over k = 0..topk-1 (routed entries only) of
 *   acc = fmaf(w[t, k], expert_out[e * max_tokens + slot(t, k), c], acc),
 * starting from +0.0f, in fp32, in ascending k (one fixed order, so that the
 * result is the same bits on every call). Enqueued on `stream`.
 */
int ll_moe_combine(void* layout, int max_tokens, int num_tokens, int hidden,
                   int num_experts, int topk, int dtype, int parity,
                   const void* expert_out, const int32_t* topk_idx,
                   const float* topk_weights, float* out, hipStream_t stream);

/*
 * Two-phase combine: the combine as a put from the expert side followed by a
 * wait-and-fold on the token side, the form a combine takes when expert and
 * token live on different devices.
 *   - rocSHMEM example "LL_MoE/LL_MoE_Buffers.hpp", struct LLMoEBuffer: the
 *     combine send and receive buffers ([num_experts * num_tokens,
 *     hidden + 1], bf16 payload) and the int64 combine flag per expert; the
 *     pointer table of LLMoEBufferLayout aliases them to the dispatch buffers
 *     of the same set, and clean_meta() treats count and flag as one array.
 *   - mscclpp "mscclpp.h", comment above struct mscclppDevConn: the data is
 *     put first and signalled after; the receiver reads it only after the
 *     signal.
 *   - memra-engine "src/tp_ar.rs": the fold of staged data is ordered after
 *     the peer's push (memra_tp_ar_fold), and a device wait is bounded and
 *     leaves a refusal code when it runs out (memra_tp_ar_1stage).
 * On one GPU the put is a local copy: the combine message of token t from
 * expert e is staged at row e * max_tokens + t of set q's combine send
 * buffer (= its send buffer, spent once the dispatch of set q is complete),
 * and expert e's flag is the high 32 bits of signal word e of set q. The
 * dispatch's count sits in the low 32 bits; the flag is up once
 * high == low. Neither call resets the flags: the next launch of parity 1-q
 * zeroes set q, as for the counts.
 * Both calls need hidden % 8 == 0, a combine message of at most
 * LL_MOE_MAX_MESSAGE_BYTES (hidden <= 22520), num_experts <=
 * LL_MOE_SEND_MAX_EXPERTS, num_experts * max_tokens < 2^31, and at most one
 * pick per (token, expert) in the routing (two picks of one expert would
 * share one staging row). Neither writes outside the regions it names.
 */
#define LL_MOE_SEND_MAX_EXPERTS 4096
#define LL_MOE_REFUSAL_FLAG_WAIT 1
#define LL_MOE_RECV_READY 0x100
/* Set beside LL_MOE_RECV_READY when the waiting workgroup's first look
 * found the set incomplete: the call started before the work it waits for
 * had finished (it overlapped with it). Informational only. */
#define LL_MOE_RECV_WAITED 0x200

/*
 * ll_moe_combine_send — expert side: stage every received message's output
 * and raise the flags of set `parity`.
 *   layout:     device, as for dispatch. Read: the low halves of set q's
 *               signal words (the dispatch counts) and the int32 headers of
 *               set q's receive rows. Written: set q's send buffer (staging
 *               rows only), the high halves of set q's signal words, and set
 *               1-q's signal words (zeroed).
 *   expert_out: device, bf16 [num_experts * max_tokens, hidden], 16-byte
 *               aligned, in receive-slot order as for ll_moe_combine.
 * For every expert e and j < count_e (count_e = low half of signal word e,
 * taken as max_tokens if larger), with t = the header of receive row
 * e * max_tokens + j: staging row e * max_tokens + t, at send_q +
 * (e * max_tokens + t) * mc, := int32 t, then the bits of expert_out row
 * e * max_tokens + j. Then the high half of signal word e is raised by the
 * number of rows staged for e, with device-scope release semantics after
 * those rows. A header outside [0, max_tokens) stages nothing, so that
 * expert's flag never comes up.
 * Order: after the dispatch of set q and after expert_out is written
 * (stream order or events). expert_out may not overlap the layout.
 * Enqueued on `stream`.
 */
int ll_moe_combine_send(void* layout, int max_tokens, int hidden, int num_experts,
                        int dtype, int parity, const void* expert_out,
                        hipStream_t stream);

/*
 * ll_moe_combine_recv — token side: wait for the experts' flags, then fold
 * the staged rows.
 *   layout:       device, as for dispatch. Read: set q's signal words and
 *                 staging rows. Written: set 1-q's signal words (zeroed).
 *   topk_idx:     device, int32 [num_tokens, topk] (the dispatch routing;
 *                 an entry outside [0, num_experts) is masked).
 *   topk_weights: device, fp32 [num_tokens, topk].
 *   out:          device, fp32 [num_tokens, hidden], 16-byte aligned; may
 *                 not overlap the layout.
 *   max_spins:    >= 1; polls of the flags before the wait gives up.
 *   status:       device, int32, 4-byte aligned, zeroed by the caller. One
 *                 workgroup polls the flags and posts the outcome here for
 *                 the others: LL_MOE_RECV_READY once every expert's flag is
 *                 up (an expert that received nothing is up), with
 *                 LL_MOE_RECV_WAITED beside it when a flag was still down at
 *                 the first look;
 *                 LL_MOE_REFUSAL_FLAG_WAIT set when a wait ran out, and out
 *                 is then unspecified. Every wait is bounded, so the launch
 *                 always ends.
 * out[t, c] = fma chain over the routed k in ascending order, from +0.0f,
 * of acc = fmaf(w[t, k], bf16 column c of staging row e * max_tokens + t,
 * acc), in fp32: the same expression, and so the same bits, as
 * ll_moe_combine on the same routing and expert outputs.
 * Order: after the dispatch of set q (its counts must be final); it may be
 * enqueued on another stream before ll_moe_combine_send of set q runs and
 * then waits for its flags (its grid is bounded, 512 workgroups, so that it
 * leaves the expert side room to run). Enqueued on `stream`.
 */
int ll_moe_combine_recv(void* layout, int max_tokens, int num_tokens, int hidden,
                        int num_experts, int topk, int dtype, int parity,
                        const int32_t* topk_idx, const float* topk_weights, float* out,
                        int max_spins, int32_t* status, hipStream_t stream);

/*
 * ll_moe_dispatch_recv — expert side of the dispatch of set `parity`: wait
 * until the set's messages are complete, then unpack them into the arrays
 * an expert's matrix product reads.
 *   - rocSHMEM example "LL_MoE/LL_MoE_Buffers.hpp", struct LLMoEBuffer: the
 *     receive rows [num_experts * num_tokens, hidden + 1] and the int64
 *     per-expert count.
 *   - mscclpp "mscclpp.h", comment above struct mscclppDevConn: the
 *     receiver reads only after the signal.
 *   - memra-engine "src/tp_ar.rs", memra_tp_ar_1stage: a device wait is
 *     bounded and leaves a refusal code when it runs out.
 * Set q is complete once its counts (the low halves of its signal words,
 * each taken as max_tokens if larger) add up to `expected`, the number of
 * messages the step routes (num_tokens * topk less masked entries): a
 * partial count does not tell which of an expert's slots are written, the
 * sum does. Then, for every expert e and j < count_e, receive row
 * r = e * max_tokens + j gives:
 *   payload row r := the message's payload without its header (bf16: the
 *     2 * hidden bytes of x[t]; fp8: the hidden e4m3 codes);
 *   scales row r  := fp8 only: its hidden / 128 fp32 scales;
 *   src_tokens[r] := its int32 header t;
 *   counts[e]     := count_e.
 * Rows at or past count_e are not written; bytes move unchanged.
 *   layout:     device, as for dispatch. Read: set q's signal words and
 *               receive rows. Written: set 1-q's signal words (zeroed).
 *   expected:   0 <= expected <= num_experts * max_tokens.
 *   payload:    device, [num_experts * max_tokens, row] with row = 2*hidden
 *               (bf16) or hidden (fp8) bytes, 16-byte aligned.
 *   scales:     device, fp32 [num_experts * max_tokens, hidden / 128],
 *               4-byte aligned; fp8 only (ignored for bf16, may be NULL).
 *   src_tokens: device, int32 [num_experts * max_tokens].
 *   counts:     device, int32 [num_experts].
 *   max_spins:  >= 1; polls of the counts before the wait gives up.
 *   status:     device, int32, 4-byte aligned, zeroed by the caller. One
 *               workgroup polls the counts and posts the outcome here for
 *               the others: LL_MOE_RECV_READY once the counts have added
 *               up (with LL_MOE_RECV_WAITED beside it when they had not at
 *               the first look); LL_MOE_REFUSAL_COUNT_WAIT set when a wait ran out (the
 *               outputs are then unspecified). Every wait is bounded.
 * An `expected` other than the routed count is a caller error: too large,
 * the wait runs out; too small, the unpack may start early and its outputs
 * are unspecified (every access stays inside the arrays described here).
 * No output may overlap the layout. The call may be enqueued on another
 * stream before the dispatch of set q completes (it then waits for it),
 * but after every earlier launch that cleans or reads set q. If it holds
 * the GPU resources the dispatch needs to run, the wait runs out into a
 * refusal. Requires num_experts <= LL_MOE_SEND_MAX_EXPERTS and
 * num_experts * max_tokens < 2^31. Enqueued on `stream`.
 */
#define LL_MOE_REFUSAL_COUNT_WAIT 2
int ll_moe_dispatch_recv(void* layout, int max_tokens, int hidden, int num_experts,
                         int dtype, int parity, int expected, void* payload, float* scales,
                         int32_t* src_tokens, int32_t* counts, int max_spins,
                         int32_t* status, hipStream_t stream);

/*
 * ll_moe_clean_signals — zero the num_experts int64 signal words of set
 * `parity` (the rocSHMEM example's clean_meta(): the dispatch count words
 * and the combine flag words are one array). Enqueued on `stream`.
 */
int ll_moe_clean_signals(void* layout, int max_tokens, int hidden,
                         int num_experts, int dtype, int parity,
                         hipStream_t stream);

/* Name of a status code (static string). */
const char* ll_moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LL_MOE_H_ */
