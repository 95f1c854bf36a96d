// Host-side argument checks shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "plan.hpp"
#include "spec_verify.h"

namespace sv {

inline bool is_aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline int elems_per_vec(int dtype) { return dtype == SPEC_BF16 ? 8 : 4; }
inline size_t elem_bytes(int dtype) { return dtype == SPEC_BF16 ? 2 : 4; }

inline int check_dims(int B, int K, int V) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 2 || V > SPEC_MAX_V) return SPEC_ERR_ARG;
  return SPEC_OK;
}

inline int check_dtype(int dtype) {
  return (dtype == SPEC_F32 || dtype == SPEC_BF16) ? SPEC_OK : SPEC_ERR_DTYPE;
}

inline int check_logits(const void* p, int dtype) {
  return (p != nullptr && is_aligned(p, elem_bytes(dtype))) ? SPEC_OK : SPEC_ERR_ARG;
}

// The workspace must hold at least spec_workspace_bytes for the call's sizes; its halves then
// hold this shape's words and data whatever size it was allocated for.
inline int check_workspace(const void* ws, size_t bytes, int B, int K, int V, int F) {
  if (ws == nullptr || !is_aligned(ws, 256)) return SPEC_ERR_WORKSPACE;
  const WsLayout L = ws_layout(B, K, V, F, bytes);
  if (bytes < L.total || !L.fits) return SPEC_ERR_WORKSPACE;
  return SPEC_OK;
}

inline bool grid_fits(size_t blocks) { return blocks >= 1 && blocks <= 0x7fffffffull; }

// log2(e) / T, the factor that turns a logit into a base-2 exponent at temperature T
inline float exp2_scale(float T) {
  return static_cast<float>(1.4426950408889634074 / static_cast<double>(T));
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

template <typename T>
inline T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Greedy verification with optional draft lengths and p/q outputs (defined with the greedy
// kernel); the point-mass verification entry uses it at temperature zero.
int greedy_point_entry(const void* target, int dtype, const int32_t* xtok, const int32_t* dlen,
                       const int32_t* kv_in, int B, int K, int V, int32_t* out_tok,
                       int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                       size_t ws_bytes, hipStream_t stream);

}  // namespace sv
