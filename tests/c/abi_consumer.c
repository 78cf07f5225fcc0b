/*
 * A plain C99 consumer of the C ABI (include/ll_moe.h): no Python, no
 * PyTorch, only the HIP runtime API for device memory. Test infrastructure:
 * it links the oracle to check the library's results.
 *
 *   abi_consumer host   layout sizes and offsets against the oracle, status
 *                       strings, and argument errors caught before any
 *                       launch (no GPU needed)
 *   abi_consumer gpu    dispatch and combine of a small seeded batch, both
 *                       parities, bf16 and fp8 payloads, on the GPU; the
 *                       whole layout byte for byte and the combine output
 *                       bit for bit against the oracle; then, on routings
 *                       with distinct experts per token, the expert side
 *                       (ll_moe_dispatch_recv: payload, scales, sources and
 *                       counts byte for byte) and the two-phase combine
 *                       (ll_moe_combine_send / _recv: layout and output)
 * Prints "ok" and exits 0 on success; prints the first mismatch and exits 1
 * otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ll_moe.h"

/* the oracle's C entry points (oracle/ll_moe_oracle.c) */
int oracle_layout(int max_tokens, int hidden, int num_experts, int dtype, uint64_t out[7]);
int oracle_dispatch(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                    int num_experts, int topk, int dtype, int parity, const uint16_t* x,
                    const int32_t* idx);
int oracle_combine(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                   int num_experts, int topk, int dtype, int parity,
                   const uint16_t* expert_out, const int32_t* idx, const float* weights,
                   float* out);
int oracle_clean(uint8_t* image, int max_tokens, int hidden, int num_experts, int dtype,
                 int parity);
int oracle_route(int num_tokens, int topk, int num_experts, int max_tokens, const int32_t* idx,
                 int32_t* slot, int64_t* cnt);
int oracle_combine_send(uint8_t* image, int max_tokens, int hidden, int num_experts, int dtype,
                        int parity, const uint16_t* expert_out);
int oracle_combine_recv(uint8_t* image, int max_tokens, int num_tokens, int hidden,
                        int num_experts, int topk, int dtype, int parity, const int32_t* idx,
                        const float* weights, float* out);
int oracle_dispatch_recv(uint8_t* image, int max_tokens, int hidden, int num_experts, int dtype,
                         int parity, int expected, uint8_t* payload, float* scales, int32_t* src,
                         int32_t* counts);

static int fail(const char* what) {
  printf("FAIL: %s\n", what);
  return 1;
}

/* 64-bit LCG (Knuth's MMIX constants), top 32 bits out */
static uint64_t lcg_state = 12345;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg_state >> 32);
}
static uint16_t bf16_of_unit(void) { /* a number in [-2, 2), bf16 by truncation */
  float f = ((float)lcg() / 4294967296.0f) * 4.0f - 2.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int host_checks(void) {
  static const int shapes[][4] = {{128, 7168, 256, 0}, {128, 7168, 256, 1}, {40, 1032, 17, 0},
                                  {1024, 7168, 256, 0}, {3, 128, 5, LL_MOE_FP8_E4M3}};
  for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const int* s = shapes[i];
    uint64_t lay[7];
    size_t bytes = 0, send = 0, recv = 0, sig = 0, md = 0;
    if (oracle_layout(s[0], s[1], s[2], s[3], lay) != 0) return fail("oracle layout");
    if (ll_moe_layout_bytes(s[0], s[1], s[2], s[3], &bytes) != LL_MOE_SUCCESS)
      return fail("layout bytes");
    if (bytes != lay[0]) return fail("layout bytes differ from the oracle");
    for (int q = 0; q < 2; ++q) {
      if (ll_moe_layout_offsets(s[0], s[1], s[2], s[3], q, &send, &recv, &sig, &md) !=
          LL_MOE_SUCCESS)
        return fail("layout offsets");
      if (send != lay[1 + q] || recv != lay[3 + q] || sig != lay[5 + q])
        return fail("layout offsets differ from the oracle");
    }
  }
  if (strcmp(ll_moe_status_string(LL_MOE_SUCCESS), "LL_MOE_SUCCESS") != 0)
    return fail("status string");
  /* argument errors: found before anything is enqueued (no device needed) */
  void* fake = (void*)(uintptr_t)0x100000;
  if (ll_moe_dispatch(fake, 128, 128, 7168, 256, 8, 0, 2, fake, fake, NULL) !=
      LL_MOE_INVALID_ARGUMENT)
    return fail("parity 2 accepted");
  if (ll_moe_dispatch(fake, 128, 129, 7168, 256, 8, 0, 0, fake, fake, NULL) !=
      LL_MOE_INVALID_ARGUMENT)
    return fail("num_tokens above max_tokens accepted");
  if (ll_moe_combine(fake, 128, 128, 7168, 256, 300, 0, 0, fake, fake, fake, fake, NULL) !=
      LL_MOE_INVALID_ARGUMENT)
    return fail("topk above num_experts accepted");
  if (ll_moe_clean_signals(NULL, 128, 7168, 256, 0, 0, NULL) != LL_MOE_INVALID_ARGUMENT)
    return fail("null layout accepted");
  return 0;
}

#define HIPCHECK(x)                                  \
  do {                                               \
    if ((x) != hipSuccess) return fail(#x);          \
  } while (0)

static int gpu_checks(int dtype) {
  enum { N = 37, CAP = 40, H = 384, E = 9, K = 3 };
  size_t total = 0;
  if (ll_moe_layout_bytes(CAP, H, E, dtype, &total) != LL_MOE_SUCCESS) return fail("layout");
  uint16_t* x = malloc((size_t)N * H * 2);
  int32_t* idx = malloc((size_t)N * K * 4);
  float* w = malloc((size_t)N * K * 4);
  uint16_t* y = malloc((size_t)E * CAP * H * 2);
  float* out = malloc((size_t)N * H * 4);
  float* ref = malloc((size_t)N * H * 4);
  uint8_t* image = malloc(total);
  uint8_t* got = malloc(total);
  if (!x || !idx || !w || !y || !out || !ref || !image || !got) return fail("host memory");
  for (int i = 0; i < N * H; ++i) x[i] = bf16_of_unit();
  for (int i = 0; i < N * K; ++i) {
    const uint32_t r = lcg();
    idx[i] = (r & 31) == 0 ? -1 : (int32_t)(r % E); /* repeats and masked entries */
    w[i] = (float)(lcg() >> 8) / 16777216.0f;
  }
  for (size_t i = 0; i < (size_t)E * CAP * H; ++i) y[i] = bf16_of_unit();

  void *d_lay, *d_x, *d_idx, *d_w, *d_y, *d_out;
  HIPCHECK(hipMalloc(&d_lay, total));
  HIPCHECK(hipMalloc(&d_x, (size_t)N * H * 2));
  HIPCHECK(hipMalloc(&d_idx, (size_t)N * K * 4));
  HIPCHECK(hipMalloc(&d_w, (size_t)N * K * 4));
  HIPCHECK(hipMalloc(&d_y, (size_t)E * CAP * H * 2));
  HIPCHECK(hipMalloc(&d_out, (size_t)N * H * 4));
  HIPCHECK(hipMemset(d_lay, 0xA5, total));
  HIPCHECK(hipMemcpy(d_x, x, (size_t)N * H * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_idx, idx, (size_t)N * K * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_w, w, (size_t)N * K * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_y, y, (size_t)E * CAP * H * 2, hipMemcpyHostToDevice));
  memset(image, 0xA5, total);

  for (int q = 0; q < 2; ++q) {
    if (ll_moe_clean_signals(d_lay, CAP, H, E, dtype, q, NULL) != LL_MOE_SUCCESS)
      return fail("clean");
    oracle_clean(image, CAP, H, E, dtype, q);
  }
  for (int q = 0; q < 2; ++q) {
    if (ll_moe_dispatch(d_lay, CAP, N, H, E, K, dtype, q, d_x, d_idx, NULL) != LL_MOE_SUCCESS)
      return fail("dispatch");
    if (ll_moe_combine(d_lay, CAP, N, H, E, K, dtype, q, d_y, d_idx, d_w, d_out, NULL) !=
        LL_MOE_SUCCESS)
      return fail("combine");
    HIPCHECK(hipDeviceSynchronize());
    if (oracle_dispatch(image, CAP, N, H, E, K, dtype, q, x, idx) != 0) return fail("oracle");
    if (oracle_combine(image, CAP, N, H, E, K, dtype, q, y, idx, w, ref) != 0)
      return fail("oracle combine");
    HIPCHECK(hipMemcpy(got, d_lay, total, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(out, d_out, (size_t)N * H * 4, hipMemcpyDeviceToHost));
    for (size_t b = 0; b < total; ++b)
      if (got[b] != image[b]) {
        printf("FAIL: dtype %d parity %d: layout byte %zu is %02x, the oracle's %02x\n", dtype,
               q, b, got[b], image[b]);
        return 1;
      }
    if (memcmp(out, ref, (size_t)N * H * 4) != 0) return fail("combine bits differ");
  }
  /* the expert side and the two-phase combine: at most one pick per
   * (token, expert), some picks masked */
  for (int t = 0; t < N; ++t) {
    const int first = (int)(lcg() % E);
    for (int k = 0; k < K; ++k)
      idx[t * K + k] = (lcg() & 15) == 0 ? -1 : (first + 2 * k) % E;
  }
  HIPCHECK(hipMemcpy(d_idx, idx, (size_t)N * K * 4, hipMemcpyHostToDevice));
  {
    int32_t slot[N * K];
    int64_t cnt[E];
    if (oracle_route(N, K, E, CAP, idx, slot, cnt) != 0) return fail("oracle route");
    int expected = 0;
    for (int e = 0; e < E; ++e) expected += (int)cnt[e];
    const size_t rows = (size_t)E * CAP;
    const size_t pb = dtype == LL_MOE_BF16 ? 2 * (size_t)H : (size_t)H;
    const size_t ns = dtype == LL_MOE_BF16 ? 1 : (size_t)H / 128;
    uint8_t* pay = malloc(rows * pb);
    uint8_t* pay_ref = malloc(rows * pb);
    float* sc = malloc(rows * ns * 4);
    float* sc_ref = malloc(rows * ns * 4);
    int32_t* src = malloc(rows * 4);
    int32_t* src_ref = malloc(rows * 4);
    int32_t counts[E], counts_ref[E], status = 0;
    if (!pay || !pay_ref || !sc || !sc_ref || !src || !src_ref) return fail("host memory");
    void *d_pay, *d_sc, *d_src, *d_cnt, *d_status;
    HIPCHECK(hipMalloc(&d_pay, rows * pb));
    HIPCHECK(hipMalloc(&d_sc, rows * ns * 4));
    HIPCHECK(hipMalloc(&d_src, rows * 4));
    HIPCHECK(hipMalloc(&d_cnt, E * 4));
    HIPCHECK(hipMalloc(&d_status, 4));
    for (int q = 0; q < 2; ++q) {
      /* outputs start as the same sentinel on both sides */
      memset(pay_ref, 0x5A, rows * pb);
      memset(sc_ref, 0x5A, rows * ns * 4);
      memset(src_ref, 0x5A, rows * 4);
      HIPCHECK(hipMemset(d_pay, 0x5A, rows * pb));
      HIPCHECK(hipMemset(d_sc, 0x5A, rows * ns * 4));
      HIPCHECK(hipMemset(d_src, 0x5A, rows * 4));
      HIPCHECK(hipMemset(d_status, 0, 4));
      if (ll_moe_dispatch(d_lay, CAP, N, H, E, K, dtype, q, d_x, d_idx, NULL) != LL_MOE_SUCCESS)
        return fail("dispatch (two-phase)");
      if (ll_moe_dispatch_recv(d_lay, CAP, H, E, dtype, q, expected, d_pay,
                               dtype == LL_MOE_BF16 ? NULL : (float*)d_sc, (int32_t*)d_src,
                               (int32_t*)d_cnt, 1 << 20, (int32_t*)d_status,
                               NULL) != LL_MOE_SUCCESS)
        return fail("dispatch_recv");
      if (ll_moe_combine_send(d_lay, CAP, H, E, dtype, q, d_y, NULL) != LL_MOE_SUCCESS)
        return fail("combine_send");
      HIPCHECK(hipDeviceSynchronize());
      HIPCHECK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
      if ((status & ~LL_MOE_RECV_WAITED) != LL_MOE_RECV_READY) return fail("dispatch_recv status");
      HIPCHECK(hipMemset(d_status, 0, 4));
      if (ll_moe_combine_recv(d_lay, CAP, N, H, E, K, dtype, q, d_idx, d_w, d_out, 1 << 20,
                              (int32_t*)d_status, NULL) != LL_MOE_SUCCESS)
        return fail("combine_recv");
      HIPCHECK(hipDeviceSynchronize());
      HIPCHECK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
      if ((status & ~LL_MOE_RECV_WAITED) != LL_MOE_RECV_READY) return fail("combine_recv status");

      if (oracle_dispatch(image, CAP, N, H, E, K, dtype, q, x, idx) != 0) return fail("oracle");
      if (oracle_dispatch_recv(image, CAP, H, E, dtype, q, expected, pay_ref,
                               dtype == LL_MOE_BF16 ? NULL : sc_ref, src_ref, counts_ref) != 0)
        return fail("oracle dispatch_recv");
      if (oracle_combine_send(image, CAP, H, E, dtype, q, y) != 0) return fail("oracle send");
      if (oracle_combine_recv(image, CAP, N, H, E, K, dtype, q, idx, w, ref) != 0)
        return fail("oracle recv");
      HIPCHECK(hipMemcpy(pay, d_pay, rows * pb, hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(sc, d_sc, rows * ns * 4, hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(src, d_src, rows * 4, hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(counts, d_cnt, E * 4, hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(got, d_lay, total, hipMemcpyDeviceToHost));
      HIPCHECK(hipMemcpy(out, d_out, (size_t)N * H * 4, hipMemcpyDeviceToHost));
      if (memcmp(pay, pay_ref, rows * pb) != 0) return fail("unpacked payload differs");
      if (dtype != LL_MOE_BF16 && memcmp(sc, sc_ref, rows * ns * 4) != 0)
        return fail("unpacked scales differ");
      if (memcmp(src, src_ref, rows * 4) != 0) return fail("unpacked sources differ");
      if (memcmp(counts, counts_ref, E * 4) != 0) return fail("unpacked counts differ");
      if (memcmp(got, image, total) != 0) return fail("two-phase layout differs");
      if (memcmp(out, ref, (size_t)N * H * 4) != 0) return fail("two-phase combine bits differ");
    }
    hipFree(d_pay), hipFree(d_sc), hipFree(d_src), hipFree(d_cnt), hipFree(d_status);
    free(pay), free(pay_ref), free(sc), free(sc_ref), free(src), free(src_ref);
  }
  hipFree(d_lay);
  hipFree(d_x);
  hipFree(d_idx);
  hipFree(d_w);
  hipFree(d_y);
  hipFree(d_out);
  free(x), free(idx), free(w), free(y), free(out), free(ref), free(image), free(got);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage: abi_consumer host|gpu");
  int rc;
  if (strcmp(argv[1], "gpu") == 0)
    rc = gpu_checks(LL_MOE_BF16) || gpu_checks(LL_MOE_FP8_E4M3);
  else
    rc = host_checks();
  if (rc == 0) printf("ok\n");
  return rc;
}
