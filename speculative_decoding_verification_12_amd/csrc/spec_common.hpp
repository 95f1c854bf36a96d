// Device helpers shared by the verification kernels (gfx950, wave64).
//
// Every logit row is streamed once with 16-byte vector loads. A row is split into a scalar head
// (elements before its first 16-byte boundary), whole vectors, and a scalar tail, so any V and
// any row alignment work; chunks of a row are ranges of whole vectors, chunk 0 also owns the
// head and the last chunk the tail, which keeps chunk order equal to token order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace sv {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr double kLn2 = 0.69314718055994530941723212145818;

// ------------------------------------------------------------------------------ element types
template <typename TIn> struct Elem;

// bfloat16 stored as its 16-bit pattern; 8 per 16-byte vector
template <> struct Elem<uint16_t> {
  static constexpr int N = 8;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;   // two bf16 -inf
  __device__ static __forceinline__ float one(const uint16_t* p, int i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  // element j of a vector stored as 32-bit words (e.g. in LDS)
  __device__ static __forceinline__ float from_words(const uint32_t* w, int j) {
    const uint32_t x = w[j >> 1];
    return __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  __device__ static __forceinline__ void unpack(const uint4& q, float* v) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
};

template <> struct Elem<float> {
  static constexpr int N = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ static __forceinline__ float one(const float* p, int i) { return p[i]; }
  __device__ static __forceinline__ float from_words(const uint32_t* w, int j) {
    return __uint_as_float(w[j]);
  }
  __device__ static __forceinline__ void unpack(const uint4& q, float* v) {
    v[0] = __uint_as_float(q.x);
    v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z);
    v[3] = __uint_as_float(q.w);
  }
};

template <typename TIn>
__device__ __forceinline__ uint4 neg_inf_vec() {
  const uint32_t w = Elem<TIn>::kNegInfWord;
  return make_uint4(w, w, w, w);
}

// 2^x on the hardware exponential unit (results below 2^-126 may flush to zero, which is far
// below the resolution any sum here can see)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------------ row layout
struct RowSpan {
  int head;   // elements [0, head) precede the first 16-byte boundary
  int nvec;   // whole vectors after the head
  int tail;   // first element after the vectors; [tail, V) is the scalar tail
};

template <typename TIn>
__device__ __forceinline__ RowSpan row_span(const TIn* row, int V) {
  constexpr int N = Elem<TIn>::N;
  const unsigned mis = static_cast<unsigned>(reinterpret_cast<uintptr_t>(row) & 15u);
  int head = static_cast<int>(((16u - mis) & 15u) / sizeof(TIn));
  if (head > V) head = V;
  const int nvec = (V - head) / N;
  return RowSpan{head, nvec, head + nvec * N};
}

// vector range [vbeg, vend) of chunk `ch` of a row with span `sp`
struct ChunkRange {
  int vbeg, vend;
  bool first, last;
};

__device__ __forceinline__ ChunkRange chunk_range(const RowSpan& sp, int ch, int nchunk, int cv) {
  ChunkRange c;
  c.vbeg = min(ch * cv, sp.nvec);
  c.vend = min(c.vbeg + cv, sp.nvec);
  c.first = ch == 0;
  c.last = ch == nchunk - 1;
  return c;
}

// ------------------------------------------------------------------------------ wave reductions
// xor-butterfly reductions: every lane ends with the same value, combined in a fixed order, so
// results are deterministic run to run.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

// reductions inside aligned segments of `width` lanes (a power of two <= 64)
__device__ __forceinline__ float seg_max(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double seg_sum(double v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (value, index) ordered by value descending, then index ascending
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// inclusive prefix sum over the 64 lanes in lane order
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// ------------------------------------------------------------------------------ arrival
// Workgroups of one group (a request or a row) publish partial results and count themselves in;
// the last to arrive merges them. The eight XCDs have separate L2 caches, so the partials are
// written and read with device-scope (agent) atomic stores/loads, which are coherent across
// XCDs by themselves; no L2 writeback or invalidate is needed. A device-scope __threadfence()
// would write back the whole L2 of the XCD for every workgroup, which serialises thousands of
// small workgroups.
__device__ __forceinline__ void store_coherent(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ uint64_t load_coherent(const void* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(static_cast<const uint64_t*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return static_cast<uint64_t>(__float_as_uint(a)) |
         (static_cast<uint64_t>(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ uint64_t pack2(float a, int b) {
  return pack2(a, __int_as_float(b));
}
__device__ __forceinline__ float lo_float(uint64_t x) {
  return __uint_as_float(static_cast<uint32_t>(x));
}
__device__ __forceinline__ float hi_float(uint64_t x) {
  return __uint_as_float(static_cast<uint32_t>(x >> 32));
}
__device__ __forceinline__ int hi_int(uint64_t x) { return static_cast<int>(x >> 32); }
__device__ __forceinline__ uint64_t dbits(double d) {
  return static_cast<uint64_t>(__double_as_longlong(d));
}
__device__ __forceinline__ double bits_d(uint64_t x) {
  return __longlong_as_double(static_cast<long long>(x));
}

// Counts this workgroup in; true (in every thread) for the last of `expected` to arrive. Every
// wave first waits for its own memory operations (the coherent partial stores among them) to
// complete, so when the counter moves, this workgroup's partials are at the device coherence
// point; the last workgroup then reads them with load_coherent.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == expected - 1u) ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sv
