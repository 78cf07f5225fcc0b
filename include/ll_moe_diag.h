/*
 * ll_moe_diag.h — diagnostic entry points of libllmoe.so. Not part of the
 * dispatch / combine step: one exposes a device building block so that tests
 * can compare it with an independent implementation, the other is a
 * concurrent reader of the dispatch's counts.
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
 * ll_moe_diag_watch — a concurrent consumer of a bf16 dispatch's counts, for
 * testing the publish order of ll_moe_dispatch: a count is raised only after
 * the messages it counts are visible at device scope (mscclpp.h, the comment
 * above struct mscclppDevConn: data first, then the signal; the receiver
 * reads data only after it has seen the signal). Enqueue it on one stream
 * while a dispatch with the same arguments runs on another. Up to 64
 * workgroups, each owning a subset of the experts, repeatedly load their
 * experts' counts of set `parity` with acquire semantics at device scope
 * and, for each expert, count the receive rows the routing will fill whose
 * header names a token routed to that expert and whose sampled payload words
 * equal that token's row of x. An expert whose acquired count exceeds the
 * rows found is a violation. A workgroup stops when its acquired counts
 * reach its experts' routed messages, or after max_passes passes.
 *   layout ... topk_idx: as for ll_moe_dispatch with dtype LL_MOE_BF16; the
 *     receive rows should hold a pattern that is no message (a header
 *     outside [0, num_tokens)) and the counts of set `parity` should be 0.
 *   max_passes: >= 1; bounds the run, which therefore always ends.
 *   report: device, int64[4], zero on entry; receives the largest number
 *     of passes of a workgroup, the number of passes (over all workgroups)
 *     whose acquired total was strictly between 0 and the workgroup's
 *     routed total, the number of violations, and the sum of the last
 *     acquired totals.
 * num_experts at most 2048. Returns an ll_moe_status_t (INVALID_ARGUMENT as
 * for ll_moe_dispatch, and for a larger num_experts, max_passes < 1 or a
 * null or misaligned report).
 */
int ll_moe_diag_watch(const void* layout, int max_tokens, int num_tokens, int hidden,
                      int num_experts, int topk, int parity, const void* x,
                      const int32_t* topk_idx, int max_passes, long long* report,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LL_MOE_DIAG_H_ */
