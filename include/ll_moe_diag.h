/*
 * ll_moe_diag.h — diagnostic entry points of libllmoe.so. Not part of the
 * dispatch / combine step; they expose one of its device building blocks so
 * that tests can compare it with an independent implementation.
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

#ifdef __cplusplus
}
#endif

#endif /* LL_MOE_DIAG_H_ */
