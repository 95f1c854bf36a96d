// Device helpers shared by the verification kernels (gfx950, wave64).
//
// Every logit row is streamed once with 16-byte vector loads. A row is split into a scalar head
// (elements before its first 16-byte boundary), whole vectors, and a scalar tail, so any V and
// any row alignment work; chunks of a row are ranges of whole vectors, chunk 0 also owns the
// head and the last chunk the tail, which keeps chunk order equal to token order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
  // the stored bits, converted later with cvt (a load issued now, waited for at first use)
  __device__ static __forceinline__ uint32_t raw(const uint16_t* p, int i) { return p[i]; }
  __device__ static __forceinline__ float cvt(uint32_t r) { return __uint_as_float(r << 16); }
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
  __device__ static __forceinline__ uint32_t raw(const float* p, int i) {
    return __float_as_uint(p[i]);
  }
  __device__ static __forceinline__ float cvt(uint32_t r) { return __uint_as_float(r); }
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

// Vector i of a logit row read with a non-temporal load (the `nt` hint), for passes after which
// little or nothing of the row is read again: greedy verification (measured ~4 % faster), the
// greedy rows of mixed batches, the outcome-key statistics pass, and the sampling statistics
// pass when the call's rows exceed the Infinity Cache. Below that size the sampling statistics
// pass keeps ordinary loads, so the draw's re-read of row m hits the cache.
__device__ __forceinline__ uint4 load_stream(const uint4* p, int i) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p) + i);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// An ordinary 16-byte load of p[i] from global memory. A row pointer that reaches a load through
// a select or a struct loses its address space, and the compiler then emits a flat load, which
// the LDS wait counter also tracks; the cast keeps it a global load.
__device__ __forceinline__ uint4 load_global(const uint4* p, int i) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) v4u GlobalVec;
  const v4u t = ((GlobalVec*)p)[i];
  return make_uint4(t.x, t.y, t.z, t.w);
}

// A float2 read with one 8-byte load. Read as a float2, a pair whose .y is used only under a
// condition on .x compiles to two dependent loads (the second issued after the first returns).
__device__ __forceinline__ float2 load_f2(const float2* p) {
  const uint64_t v = *reinterpret_cast<const uint64_t*>(p);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)),
                     __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

// 2^x on the hardware exponential unit (results below 2^-126 may flush to zero, which is far
// below the resolution any sum here can see)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^((l - M) c): the weight of logit l against a reference M (a row's or a running maximum) at
// c = log2(e)/T. The difference is taken before the scaling, so the reference's own term is
// exactly 1 and a logit below it gives a value in [0, 1] at every temperature: with the product
// fl(M c) as the reference instead, its rounding error (|M c| 2^-24) becomes the exponent of the
// maximum's own term, which overflows or underflows once c is large (T below ~1e-9 at |M| ~ 10).
__device__ __forceinline__ float rel_exp2(float l, float M, float c) {
  return fast_exp2((l - M) * c);
}

// A probability 2^((l - M) c) / S with its row's normaliser folded into the exponent
// (ls = log2 S): one subtraction, one fma and one exp2 per element.
__device__ __forceinline__ float prob_exp2(float l, float M, float c, float ls) {
  return fast_exp2(fmaf(l - M, c, -ls));
}

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

// ------------------------------------------------------------------------------ DPP lane moves
// Data-parallel-primitive moves read another lane's register inside the vector ALU, with no LDS
// round trip (a ds_bpermute shuffle costs an LDS access per step). GFX9 control encodings; all
// lanes of the wave must be active where these are used.
namespace dpp {
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowShr = 0x110;        // row_shr:n is kRowShr + n (n = 1..15)
constexpr int kWaveShr1 = 0x138;      // wave_shr:1
constexpr int kRowMirror = 0x140;     // lane i of a row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141; // lane i of a half-row reads lane 7 - i
constexpr int kRowBcast15 = 0x142;    // lane 15 of each row to the whole next row
constexpr int kRowBcast31 = 0x143;    // lane 31 to rows 2 and 3
}  // namespace dpp

// Lanes outside `row_mask`, and lanes whose source is outside the row (or wave) unless
// `bound_zero`, keep `old`; with `bound_zero` such sources read as 0.
template <int ctrl, int row_mask = 0xf, bool bound_zero = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(v), ctrl, row_mask, 0xf, bound_zero));
}

template <int ctrl, int row_mask = 0xf, bool bound_zero = false>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __uint_as_float(dpp_u32<ctrl, row_mask, bound_zero>(__float_as_uint(old),
                                                             __float_as_uint(v)));
}

template <int ctrl, int row_mask = 0xf, bool bound_zero = false>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  const uint64_t o = static_cast<uint64_t>(__double_as_longlong(old));
  const uint64_t x = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = dpp_u32<ctrl, row_mask, bound_zero>(static_cast<uint32_t>(o),
                                                          static_cast<uint32_t>(x));
  const uint32_t hi = dpp_u32<ctrl, row_mask, bound_zero>(static_cast<uint32_t>(o >> 32),
                                                          static_cast<uint32_t>(x >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t x = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), lane));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Combines the lanes of every aligned group of `width` lanes (1, 2, 4, 8, 16, 32 or 64) with the
// commutative `op`; every lane of a group gets the group's result, bit for bit, because each
// step combines a lane with a partner holding the same partial of the other half.
template <typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, int width, Op op) {
  static_assert(std::is_same<T, double>::value || std::is_same<T, float>::value ||
                    std::is_same<T, int>::value,
                "double, float or int");
  auto mv = [](auto ctrl_tag, T x) -> T {
    constexpr int ctrl = decltype(ctrl_tag)::value;
    if constexpr (std::is_same<T, double>::value) return dpp_f64<ctrl>(x, x);
    else if constexpr (std::is_same<T, float>::value) return dpp_f32<ctrl>(x, x);
    else return static_cast<T>(dpp_u32<ctrl>(static_cast<uint32_t>(x), static_cast<uint32_t>(x)));
  };
  if (width >= 2) v = op(v, mv(std::integral_constant<int, dpp::kQuadXor1>{}, v));
  if (width >= 4) v = op(v, mv(std::integral_constant<int, dpp::kQuadXor2>{}, v));
  if (width >= 8) v = op(v, mv(std::integral_constant<int, dpp::kRowHalfMirror>{}, v));
  if (width >= 16) v = op(v, mv(std::integral_constant<int, dpp::kRowMirror>{}, v));
  if (width >= 32) {
    T r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (std::is_same<T, double>::value) r[i] = readlane_f64(v, 16 * i);
      else if constexpr (std::is_same<T, float>::value) r[i] = readlane_f32(v, 16 * i);
      else r[i] = static_cast<T>(__builtin_amdgcn_readlane(static_cast<int>(v), 16 * i));
    }
    const T lo = op(r[0], r[1]), hi = op(r[2], r[3]);
    const bool upper = (threadIdx.x & (kWave - 1)) >= 32;
    v = width >= 64 ? op(lo, hi) : (upper ? hi : lo);
  }
  return v;
}

struct OpAdd {
  template <typename T> __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
  __device__ double operator()(double a, double b) const { return fmax(a, b); }
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
  __device__ int operator()(int a, int b) const { return max(a, b); }
};

// Inclusive prefix sum over the 64 lanes in lane order (Hillis-Steele inside each 16-lane row,
// then the row totals carried across rows).
__device__ __forceinline__ double wave_scan_incl(double x) {
  x += dpp_f64<dpp::kRowShr + 1, 0xf, true>(0.0, x);
  x += dpp_f64<dpp::kRowShr + 2, 0xf, true>(0.0, x);
  x += dpp_f64<dpp::kRowShr + 4, 0xf, true>(0.0, x);
  x += dpp_f64<dpp::kRowShr + 8, 0xf, true>(0.0, x);
  x += dpp_f64<dpp::kRowBcast15, 0xa, false>(0.0, x);
  x += dpp_f64<dpp::kRowBcast31, 0xc, false>(0.0, x);
  return x;
}

// The previous lane's value (0 in lane 0): with an inclusive scan, the exclusive one, bit for bit.
__device__ __forceinline__ double wave_shift_up1(double x) {
  return dpp_f64<dpp::kWaveShr1, 0xf, true>(0.0, x);
}

// ------------------------------------------------------------------------------ wave reductions
// Whole-wave reductions on DPP moves: every lane ends with the same value, combined in a fixed
// order, so results are deterministic run to run.
__device__ __forceinline__ float wave_max(float v) { return group_reduce(v, kWave, OpMax{}); }
__device__ __forceinline__ float wave_sum(float v) { return group_reduce(v, kWave, OpAdd{}); }
__device__ __forceinline__ double wave_sum(double v) { return group_reduce(v, kWave, OpAdd{}); }
__device__ __forceinline__ int wave_max(int v) { return group_reduce(v, kWave, OpMax{}); }

// (value, index) ordered by value descending, then index ascending
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Wave-wide best (value, index) in that order; every lane gets it. Indices must be distinct
// among lanes with equal values (or the pairs equal), which makes the order total.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  auto step = [&](auto ctrl_tag) {
    constexpr int ctrl = decltype(ctrl_tag)::value;
    const float ov = dpp_f32<ctrl>(v, v);
    const int oi = static_cast<int>(dpp_u32<ctrl>(static_cast<uint32_t>(i), static_cast<uint32_t>(i)));
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  };
  step(std::integral_constant<int, dpp::kQuadXor1>{});
  step(std::integral_constant<int, dpp::kQuadXor2>{});
  step(std::integral_constant<int, dpp::kRowHalfMirror>{});
  step(std::integral_constant<int, dpp::kRowMirror>{});
  float bv = readlane_f32(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = readlane_f32(v, 16 * r);
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (better(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
}

// Inclusive prefix sum of ints over the 64 lanes in lane order.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += static_cast<int>(dpp_u32<dpp::kRowShr + 1, 0xf, true>(0u, static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp_u32<dpp::kRowShr + 2, 0xf, true>(0u, static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp_u32<dpp::kRowShr + 4, 0xf, true>(0u, static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp_u32<dpp::kRowShr + 8, 0xf, true>(0u, static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp_u32<dpp::kRowBcast15, 0xa, false>(0u, static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp_u32<dpp::kRowBcast31, 0xc, false>(0u, static_cast<uint32_t>(x)));
  return x;
}

// 2^x for a float64 exponent, to about 2e-7 relative: the integer part scales exactly, the
// fraction goes through the hardware exp2. x = -inf gives 0.
__device__ __forceinline__ double exp2_wide(double x) {
  if (!(x > -1074.0)) return 0.0;
  if (x >= 1024.0) return INFINITY;
  const double n = floor(x);
  return ldexp(static_cast<double>(fast_exp2(static_cast<float>(x - n))), static_cast<int>(n));
}

// ------------------------------------------------------------------------------ exchange
// Workgroups of one launch publish partial results that another workgroup of the same launch
// reads. The eight XCDs have separate L2 caches, so such words are written and read with
// device-scope (agent) atomic stores/loads, which are coherent across XCDs by themselves; no L2
// writeback or invalidate is needed. A device-scope __threadfence() would write back the whole
// L2 of the XCD for every workgroup, which serialises thousands of small workgroups.
__device__ __forceinline__ void store_coherent(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent_u32(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_coherent_u32(const void* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(static_cast<const uint32_t*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ uint64_t load_coherent(const void* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(static_cast<const uint64_t*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope compare-and-swap of a 64-bit word; returns the value found (== expected when
// the swap happened).
__device__ __forceinline__ uint64_t cas_coherent(void* p, uint64_t expected, uint64_t desired) {
  __hip_atomic_compare_exchange_strong(static_cast<uint64_t*>(p), &expected, desired,
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return expected;
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

}  // namespace sv
