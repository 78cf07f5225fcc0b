/*
 * ll_moe_diag.h — diagnostic entry points of libllmoe.so. Not part of the
 * dispatch / combine step: one exposes a device building block so that tests
 * can compare it with an independent implementation, one is a concurrent
 * reader of the dispatch's counts, and three are measurement probes that
 * move the step's bytes without the rest of its work.
 */
#ifndef LL_MOE_DIAG_H_
#define LL_MOE_DIAG_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ll_moe_diag_e4m3 — out[i] = the e4m3 code the fp8 dispatch writes for the
 * fp32 value in[i]: OCP e4m3 ("e4m3fn"), round to nearest even, finite
 * values beyond 448 and the infinities saturate to +-448 (0x7E / 0xFE),
 * every NaN gives 0x7F. The pages give no quantizer; this is the reading the
 * fp8 message of ll_moe_dispatch uses.
 *   in:  device, n fp32 values, 4-byte aligned.
 *   out: device, n bytes.
 * Enqueued on `stream`; returns an ll_moe_status_t (INVALID_ARGUMENT for a
 * null pointer with n > 0).
 */
int ll_moe_diag_e4m3(const float* in, uint8_t* out, size_t n, hipStream_t stream);

/*
 * ll_moe_diag_e4m3_in_range — the encoder of ll_moe_diag_e4m3 in the form
 * the fp8 dispatch runs for every wavefront whose blocks all have a
 * nonzero finite amax, a finite 448 / amax and no NaN: the conversion
 * without the clamp to +-448 and without the NaN patch. In such a block
 * every product x * (448 / amax) is a number of magnitude at most
 * 448 * (1 + 2^-23), and for those inputs out[i] must equal
 * ll_moe_diag_e4m3's code (values in (448, 464] round to 448). For other
 * inputs the code is whatever the conversion gives (unspecified).
 * Arguments and errors as for ll_moe_diag_e4m3.
 */
int ll_moe_diag_e4m3_in_range(const float* in, uint8_t* out, size_t n, hipStream_t stream);

/*
 * ll_moe_diag_watch — a concurrent consumer of a dispatch's counts (bf16 or
 * fp8 messages), for testing the publish order of ll_moe_dispatch: a count
 * is raised only after the messages it counts are visible at device scope
 * (mscclpp.h, the comment above struct mscclppDevConn: data first, then the
 * signal; the receiver reads data only after it has seen the signal).
 * Enqueue it on one stream while a dispatch with the same arguments runs on
 * another. Up to 64 workgroups, each owning a subset of the experts, work
 * out from the routing which token's message every slot of their experts
 * will hold (slot j of expert e: the j-th entry, in (token, pick) order,
 * naming e, below max_tokens), then repeatedly load their experts' counts
 * of set `parity` with acquire semantics at device scope and compare, whole
 * and byte for byte, the receive rows not yet found complete with the
 * expected messages. An expert whose acquired count exceeds its complete
 * rows is a violation. A workgroup stops when its acquired counts reach its
 * experts' routed messages, or after max_passes passes.
 *   layout, max_tokens, num_tokens, hidden, num_experts, topk, dtype,
 *     parity, topk_idx: as for ll_moe_dispatch; the receive rows should
 *     hold a pattern that is no message and the counts of set `parity`
 *     should be 0.
 *   messages: device, 4-byte aligned, [num_tokens, md] bytes: message(t)
 *     as ll_moe_dispatch must write it (header and payload).
 *   max_passes: >= 1; bounds the run, which therefore always ends.
 *   report: device, int64[4], zero on entry; receives the largest number
 *     of passes of a workgroup, the number of passes (over all workgroups)
 *     whose acquired total was strictly between 0 and the workgroup's
 *     routed total, the number of violations, and the sum of the last
 *     acquired totals.
 * num_experts at most 2048, num_tokens * topk at most 4096. Returns an
 * ll_moe_status_t (INVALID_ARGUMENT as for ll_moe_dispatch, and for larger
 * sizes, max_passes < 1 or a null or misaligned report or messages).
 */
int ll_moe_diag_watch(const void* layout, int max_tokens, int num_tokens, int hidden,
                      int num_experts, int topk, int dtype, int parity, const void* messages,
                      const int32_t* topk_idx, int max_passes, long long* report,
                      hipStream_t stream);

/*
 * Measurement probes. They place the step's kernels against what the part
 * itself does with the same bytes; none of them is part of the step. The
 * mscclpp.h comment above struct mscclppDevConn weighs a DMA engine's copy
 * against a copy by GPU threads; on one MI355X every byte here is moved by
 * shader loads and stores, and these probes give that path's ceilings and
 * floors. Every call enqueues one kernel on `stream` and returns an
 * ll_moe_status_t (INVALID_ARGUMENT for the cases named).
 */
#define LL_MOE_PROBE_WRITE 0  /* dst := a pattern */
#define LL_MOE_PROBE_READ 1   /* read src (one word of dst may be written) */
#define LL_MOE_PROBE_COPY 2   /* dst := src */
#define LL_MOE_PROBE_FOLD4 3  /* dst := lane-wise uint32 sum of 4 source regions */

/*
 * ll_moe_diag_stream — a contiguous stream of `bytes` bytes: write, read or
 * copy (mode above), 16-byte accesses, four in flight per thread, `blocks`
 * workgroups of 256 threads striding over the buffer; non_temporal != 0
 * gives the accesses the streaming (non-temporal) hint. FOLD4 writes
 * `bytes` bytes and reads four times as many: 16-byte chunk j of dst
 * becomes the lane-wise wrapping uint32 sum of chunk j of the four
 * consecutive `bytes`-byte regions of src, sixteen loads in flight per
 * thread. That is the combine's mix of traffic at top-k 8 (16h bytes of
 * bf16 rows read per 4h bytes of fp32 output written).
 *   dst: device, 16-byte aligned, `bytes` bytes (READ: at least 16 bytes).
 *   src: device, 16-byte aligned, `bytes` bytes (READ and COPY), 4 * `bytes`
 *        bytes (FOLD4).
 * INVALID_ARGUMENT: bytes % 16 != 0, blocks < 1, a null or misaligned
 * pointer the mode needs, an unknown mode. bytes == 0 enqueues nothing.
 */
int ll_moe_diag_stream(int mode, int non_temporal, void* dst, const void* src, size_t bytes,
                       int blocks, hipStream_t stream);

/* Cache policies of ll_moe_diag_store_rows' stores. */
#define LL_MOE_PROBE_SC1 0         /* device-coherent write-through: the dispatch's */
#define LL_MOE_PROBE_WRITE_BACK 1  /* plain stores, written back from L2 later */
#define LL_MOE_PROBE_NT 2          /* non-temporal */
#define LL_MOE_PROBE_SC1_NT 3      /* write-through and non-temporal */

/* Store routines of ll_moe_diag_store_rows. */
#define LL_MOE_PROBE_ROWS_GROUP 0   /* from LDS, each row by all threads in turn */
#define LL_MOE_PROBE_ROWS_WAVE 1    /* from LDS, each row whole by one wavefront */
#define LL_MOE_PROBE_ROWS_DIRECT 2  /* from registers, each row by all threads */

/*
 * ll_moe_diag_store_rows — the dispatch's message stores alone: row i of
 * the list receives row_bytes bytes of a pattern at base + row_offsets[i]
 * through one of the dispatch's store routines, with stores of the given
 * policy. Workgroup b (256 threads) writes rows [b * rows_per_block,
 * (b + 1) * rows_per_block):
 *   rows == LL_MOE_PROBE_ROWS_GROUP: from an LDS buffer, every row by all
 *     its threads in turn (destination-aligned 16-byte buffer stores);
 *   rows == LL_MOE_PROBE_ROWS_WAVE: from an LDS buffer, each row whole by
 *     one wavefront (wavefront w: rows w, w + 4, ...);
 *   rows == LL_MOE_PROBE_ROWS_DIRECT: straight from registers, every row by
 *     all its threads, payload chunk c at row byte 4 + 16c (dword-aligned
 *     16-byte stores at the row's own phase), as the dispatch writes its
 *     batches below 64 MiB; row_bytes must be 4 more than a multiple of 16
 *     (a message row).
 * With line != 0 the LDS routines deal the chunks to lanes by whole
 * 128-byte lines, as the dispatch does for its largest batches (ignored by
 * the direct routine). No other loads, no counts.
 *   base:        device, 16-byte aligned.
 *   row_offsets: device, int64 [nrows], each a multiple of 4; every row
 *                [offset, offset + row_bytes) must lie inside base's
 *                allocation (the caller's duty: the probe cannot see it).
 * INVALID_ARGUMENT: nrows < 0, row_bytes not a positive multiple of 4 or
 * above LL_MOE_MAX_MESSAGE_BYTES (direct: not 4 more than a multiple of
 * 16), rows_per_block outside [1, 256], an unknown routine or policy, a
 * null or misaligned pointer.
 */
int ll_moe_diag_store_rows(void* base, const int64_t* row_offsets, int nrows, int row_bytes,
                           int rows_per_block, int line, int rows, int policy,
                           hipStream_t stream);

/*
 * ll_moe_diag_gather_rows — the combine's gather alone: out[t, c] = the fma
 * chain of ll_moe_combine over k in ascending order of
 * fmaf(weights[t, k], y[rows[t, k], c], acc) from +0.0f, with the rows
 * handed in instead of computed from a routing; the combine's launch shape
 * and load forms. A row outside [0, y_rows) (a masked pick: -1) takes no
 * part.
 *   y:       device, bf16 [y_rows, hidden], 16-byte aligned.
 *   rows:    device, int32 [num_tokens, topk].
 *   weights: device, fp32 [num_tokens, topk].
 *   out:     device, fp32 [num_tokens, hidden], 16-byte aligned.
 * INVALID_ARGUMENT: num_tokens < 0, hidden not a positive multiple of 8,
 * topk outside [1, LL_MOE_MAX_TOPK], y_rows < 1 (a token with no pick in
 * range still loads row 0, its value unused), a null or misaligned
 * pointer. num_tokens == 0 enqueues nothing.
 */
int ll_moe_diag_gather_rows(const void* y, long long y_rows, int hidden, const int32_t* rows,
                            const float* weights, int num_tokens, int topk, float* out,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LL_MOE_DIAG_H_ */
