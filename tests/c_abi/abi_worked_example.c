/* Plain-C use of libspecverify through its C ABI alone: no Python, no C++ (test program).
 *
 * Case 1, greedy, bf16: the worked round of the page "LLMの生成を5倍速くする「D3D」を図で読む",
 * sections 検証のしくみ① and 検証のまとめ. Vocabulary ids 0..7 are 今日 は いい 天気 だ よ です ね;
 * the drafter proposes は いい 天気 だ よ (1 2 3 4 5); the target's top choices per row are
 * は いい 天気 です ね (1 2 3 6 7) and, for the extra row the page leaves open, 今日 (0) here.
 * Three drafts are kept, です is placed, tau = 4. With drafts 1 2 3 6 7 every draft is kept and
 * the extra row's choice follows: tau = 6.
 *
 * Case 2, sampling, fp32, K = 1, V = 2 (hand-worked, the ratio rule of the page
 * "speculative decodingとは", stages 3 and 4): target row 0 = (0, ln 3) gives p = (1/4, 3/4),
 * draft row 0 = (ln 3, 0) gives q = (3/4, 1/4), draft token 0, ratio p/q = 1/3.
 *   u0 = 0.2 < 1/3: kept; the extra row (0, 0) gives (1/2, 1/2); u1 = 0.25 draws 0, u1 = 0.75
 *   draws 1 (the smallest token whose running sum exceeds u1).
 *   u0 = 0.5: rejected; the residual max(0, p - q) = (0, 1/2) leaves only token 1.
 * Reported p_0(x_0) = 1/4, q_0(x_0) = 3/4.
 *
 * Prints "ok" and exits 0 when every output matches; prints each mismatch and exits 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "spec_verify.h"

static int failures = 0;

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

#define SPEC_OK_CALL(call)                                                          \
  do {                                                                              \
    int s_ = (call);                                                                \
    if (s_ != SPEC_OK) {                                                            \
      printf("%s failed: %s\n", #call, spec_status_string(s_));                     \
      return 2;                                                                     \
    }                                                                               \
  } while (0)

static void expect_ints(const char* what, const int32_t* got, const int32_t* want, int n) {
  for (int i = 0; i < n; ++i)
    if (got[i] != want[i]) {
      printf("FAIL %s[%d]: got %d, expected %d\n", what, i, got[i], want[i]);
      ++failures;
    }
}

static void expect_near(const char* what, float got, double want) {
  if (!(fabs((double)got - want) <= 1e-6)) {
    printf("FAIL %s: got %.9g, expected %.9g\n", what, got, want);
    ++failures;
  }
}

static int greedy_case(hipStream_t stream) {
  enum { B = 2, K = 5, V = 8 };
  /* bf16 bit patterns: 5.0 = 0x40A0, 0.0 = 0x0000 */
  const int top[K + 1] = {1, 2, 3, 6, 7, 0};
  uint16_t logits[B][K + 1][V];
  memset(logits, 0, sizeof logits);
  for (int b = 0; b < B; ++b)
    for (int k = 0; k <= K; ++k) logits[b][k][top[k]] = 0x40A0;
  const int32_t drafts[B][K] = {{1, 2, 3, 4, 5}, {1, 2, 3, 6, 7}};
  const int32_t kv_in[B] = {100, 2048};
  const int32_t want_tokens[B][K + 1] = {{1, 2, 3, 6, -1, -1}, {1, 2, 3, 6, 7, 0}};
  const int32_t want_tau[B] = {4, 6};
  const int32_t want_kv[B] = {104, 2054};

  void *d_logits, *d_drafts, *d_kv, *d_tok, *d_tau, *d_kvo, *ws;
  const size_t ws_bytes = spec_workspace_bytes(B, K, V, 1);
  HIP_OK(hipMalloc(&d_logits, sizeof logits));
  HIP_OK(hipMalloc(&d_drafts, sizeof drafts));
  HIP_OK(hipMalloc(&d_kv, sizeof kv_in));
  HIP_OK(hipMalloc(&d_tok, sizeof want_tokens));
  HIP_OK(hipMalloc(&d_tau, sizeof want_tau));
  HIP_OK(hipMalloc(&d_kvo, sizeof want_kv));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(d_logits, logits, sizeof logits, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_drafts, drafts, sizeof drafts, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_kv, kv_in, sizeof kv_in, hipMemcpyHostToDevice));
  SPEC_OK_CALL(spec_workspace_init(ws, ws_bytes, stream));
  SPEC_OK_CALL(spec_verify_greedy(d_logits, SPEC_BF16, (const int32_t*)d_drafts,
                                  (const int32_t*)d_kv, B, K, V, 0.0f, (int32_t*)d_tok,
                                  (int32_t*)d_tau, (int32_t*)d_kvo, ws, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  int32_t tok[B][K + 1], tau[B], kvo[B];
  HIP_OK(hipMemcpy(tok, d_tok, sizeof tok, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(tau, d_tau, sizeof tau, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kvo, d_kvo, sizeof kvo, hipMemcpyDeviceToHost));
  expect_ints("greedy tokens", &tok[0][0], &want_tokens[0][0], B * (K + 1));
  expect_ints("greedy tau", tau, want_tau, B);
  expect_ints("greedy kv", kvo, want_kv, B);
  hipFree(d_logits);
  hipFree(d_drafts);
  hipFree(d_kv);
  hipFree(d_tok);
  hipFree(d_tau);
  hipFree(d_kvo);
  hipFree(ws);
  return 0;
}

static int sampling_case(hipStream_t stream) {
  enum { B = 3, K = 1, V = 2 };
  const float ln3 = (float)log(3.0);
  float target[B][K + 1][V], draft[B][K][V];
  for (int b = 0; b < B; ++b) {
    target[b][0][0] = 0.0f;
    target[b][0][1] = ln3;
    target[b][1][0] = 0.0f;
    target[b][1][1] = 0.0f;
    draft[b][0][0] = ln3;
    draft[b][0][1] = 0.0f;
  }
  const int32_t drafts[B][K] = {{0}, {0}, {0}};
  const float u[B][K + 1] = {{0.2f, 0.25f}, {0.2f, 0.75f}, {0.5f, 0.9f}};
  const int32_t kv_in[B] = {7, 7, 7};
  const int32_t want_tokens[B][K + 1] = {{0, 0}, {0, 1}, {1, -1}};
  const int32_t want_tau[B] = {2, 2, 1};
  const int32_t want_kv[B] = {9, 9, 8};

  void *d_t, *d_d, *d_x, *d_u, *d_kv, *d_tok, *d_tau, *d_kvo, *d_p, *d_q, *ws;
  const size_t ws_bytes = spec_workspace_bytes(B, K, V, 1);
  HIP_OK(hipMalloc(&d_t, sizeof target));
  HIP_OK(hipMalloc(&d_d, sizeof draft));
  HIP_OK(hipMalloc(&d_x, sizeof drafts));
  HIP_OK(hipMalloc(&d_u, sizeof u));
  HIP_OK(hipMalloc(&d_kv, sizeof kv_in));
  HIP_OK(hipMalloc(&d_tok, sizeof want_tokens));
  HIP_OK(hipMalloc(&d_tau, sizeof want_tau));
  HIP_OK(hipMalloc(&d_kvo, sizeof want_kv));
  HIP_OK(hipMalloc(&d_p, sizeof(float) * B * K));
  HIP_OK(hipMalloc(&d_q, sizeof(float) * B * K));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(d_t, target, sizeof target, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_d, draft, sizeof draft, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, drafts, sizeof drafts, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_u, u, sizeof u, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_kv, kv_in, sizeof kv_in, hipMemcpyHostToDevice));
  SPEC_OK_CALL(spec_workspace_init(ws, ws_bytes, stream));
  SPEC_OK_CALL(spec_verify_sample(d_t, d_d, SPEC_F32, (const int32_t*)d_x, (const float*)d_u,
                                  (const int32_t*)d_kv, B, K, V, 1.0f, (int32_t*)d_tok,
                                  (int32_t*)d_tau, (int32_t*)d_kvo, (float*)d_p, (float*)d_q, ws,
                                  ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  int32_t tok[B][K + 1], tau[B], kvo[B];
  float p[B], q[B];
  HIP_OK(hipMemcpy(tok, d_tok, sizeof tok, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(tau, d_tau, sizeof tau, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kvo, d_kvo, sizeof kvo, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(p, d_p, sizeof p, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(q, d_q, sizeof q, hipMemcpyDeviceToHost));
  expect_ints("sampling tokens", &tok[0][0], &want_tokens[0][0], B * (K + 1));
  expect_ints("sampling tau", tau, want_tau, B);
  expect_ints("sampling kv", kvo, want_kv, B);
  for (int b = 0; b < B; ++b) {
    expect_near("p_0(x_0)", p[b], 0.25);
    expect_near("q_0(x_0)", q[b], 0.75);
  }
  hipFree(d_t);
  hipFree(d_d);
  hipFree(d_x);
  hipFree(d_u);
  hipFree(d_kv);
  hipFree(d_tok);
  hipFree(d_tau);
  hipFree(d_kvo);
  hipFree(d_p);
  hipFree(d_q);
  hipFree(ws);
  return 0;
}

int main(void) {
  if (spec_abi_version() != SPEC_ABI_VERSION) {
    printf("library ABI %d, header ABI %d\n", spec_abi_version(), SPEC_ABI_VERSION);
    return 2;
  }
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  int rc = greedy_case(stream);
  if (rc == 0) rc = sampling_case(stream);
  HIP_OK(hipStreamDestroy(stream));
  if (rc != 0) return rc;
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
