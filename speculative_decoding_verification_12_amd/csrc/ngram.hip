// Prompt-lookup drafting on gfx950 (page "speculative decodingとは", section
// "別のドラフトモデルは常に必要なのか?", the n-gram and prompt-search bullet: with no draft network,
// the engine finds a span of the prompt and of the output so far that matches the latest text
// and proposes the tokens that followed it).
//
// Rule (the readings where the page leaves the details open): the span to match is the context's
// last n tokens, n from min(n_max, L-1) down to n_min; of its earlier occurrences (start
// j <= L-n-1) the most recent is taken; the draft is the up to K tokens that follow it.
//
// For a continuation start e in [1, L-1], let r_e count how many tokens before e agree with the
// context's last tokens read backwards (ctx[e-1-i] == ctx[L-1-i] for i < r_e), capped at n_max.
// An n-token span occurs ending just before e exactly when r_e >= n, so the rule's choice (the
// longest n, then the latest start) is the largest (r_e, e) in lexicographic order with
// r_e >= n_min: a maximum over positions, packed as the 64-bit key (r_e << 32) | e.
//
// One workgroup of 1024 threads per request (a context is a few KiB to a few hundred KiB of
// token ids, a latency-bound read). The context goes through LDS in tiles of 8192 positions
// (plus the n_max tokens before each tile), all of a tile's loads in flight at once, the span's
// tokens loaded with the first tile; every thread tests 8 positions of a tile and extends the
// rare matches backwards in LDS; the workgroup reduces the keys and wave 0 copies the draft.
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

constexpr int kLookupBlock = 1024;
constexpr int kLookupWaves = kLookupBlock / kWave;
constexpr int kLookupPer = 8;                                // positions a thread tests per tile
constexpr int kLookupTile = kLookupBlock * kLookupPer;      // positions per tile
constexpr int kLookupHalo = SPEC_MAX_NGRAM;                 // tokens kept before a tile
constexpr int kLookupLoads = (kLookupHalo + kLookupTile + kLookupBlock - 1) / kLookupBlock;

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const unsigned lo = __shfl_xor(static_cast<unsigned>(v), o, kWave);
    const unsigned hi = __shfl_xor(static_cast<unsigned>(v >> 32), o, kWave);
    const unsigned long long u = (static_cast<unsigned long long>(hi) << 32) | lo;
    v = u > v ? u : v;
  }
  return v;
}

__global__ __launch_bounds__(kLookupBlock) void ngram_draft_kernel(
    const int32_t* __restrict__ ctx, long long ld, const int32_t* __restrict__ lens, int n_max,
    int n_min, int K, int32_t* __restrict__ out_tok, int32_t* __restrict__ out_len,
    int32_t* __restrict__ out_n, int32_t* __restrict__ out_src) {
  __shared__ int s_suf[SPEC_MAX_NGRAM];                  // s_suf[i] = ctx[L-1-i]
  __shared__ int s_ctx[kLookupHalo + kLookupTile];       // s_ctx[i] = ctx[e0 - halo + i]
  __shared__ unsigned long long s_best[kLookupWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int32_t* row = ctx + static_cast<size_t>(b) * static_cast<size_t>(ld);
  const int L = lens[b];
  const bool ok = L >= 0 && static_cast<long long>(L) <= ld;   // else a row error
  const int nsuf = ok ? min(n_max, L) : 0;

  unsigned long long best = 0ull;   // 0: no allowed match
  if (ok && L >= 2) {               // uniform
    // the span's own tokens, issued together with the first tile's loads
    const int sv = row[L - 1 - min(tid, nsuf - 1)];
    for (int e0 = 1; e0 < L; e0 += kLookupTile) {   // uniform
      int v[kLookupLoads];
#pragma unroll
      for (int i = 0; i < kLookupLoads; ++i) {   // clamped: every load is issued at once
        const int g = e0 - kLookupHalo + i * kLookupBlock + tid;
        v[i] = row[min(max(g, 0), L - 1)];
      }
      __syncthreads();   // the previous tile is no longer read
      if (e0 == 1 && tid < nsuf) s_suf[tid] = sv;
#pragma unroll
      for (int i = 0; i < kLookupLoads; ++i) {
        const int li = i * kLookupBlock + tid;
        if (li < kLookupHalo + kLookupTile) s_ctx[li] = v[i];
      }
      __syncthreads();
      const int last = s_suf[0];
#pragma unroll
      for (int j = 0; j < kLookupPer; ++j) {
        const int e = e0 + j * kLookupBlock + tid;   // continuation start tested
        const int li = e - e0 + kLookupHalo;          // s_ctx index of ctx[e]
        if (e < L && s_ctx[li - 1] == last) {
          int r = 1;   // ctx[e-1-r] sits at s_ctx[li-1-r], r < n_max <= halo
          while (r < n_max && r < e && s_ctx[li - 1 - r] == s_suf[r]) ++r;
          const unsigned long long key =
              (static_cast<unsigned long long>(r) << 32) | static_cast<unsigned>(e);
          if (r >= n_min && key > best) best = key;
        }
      }
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) s_best[w] = best;
  __syncthreads();
  if (w != 0) return;
  unsigned long long k2 = lane < kLookupWaves ? s_best[lane] : 0ull;
  k2 = wave_max_u64(k2);
  const int n = static_cast<int>(k2 >> 32);
  const int src = static_cast<int>(k2 & 0xffffffffull);
  const int len = !ok ? -1 : (n == 0 ? 0 : min(K, L - src));
  for (int i = lane; i < K; i += kWave)
    out_tok[static_cast<size_t>(b) * K + i] = i < len ? row[src + i] : -1;
  if (lane == 0) {
    out_len[b] = len;
    if (out_n) out_n[b] = n;
    if (out_src) out_src[b] = n > 0 ? src : -1;
  }
}

}  // namespace
}  // namespace sv

extern "C" int spec_ngram_draft(const int32_t* context, long long ld, const int32_t* context_len,
                                int B, int n_max, int n_min, int K, int32_t* out_tokens,
                                int32_t* out_len, int32_t* out_ngram, int32_t* out_src,
                                hipStream_t stream) {
  using namespace sv;
  if (context == nullptr || context_len == nullptr || out_tokens == nullptr ||
      out_len == nullptr || B < 1 || ld < 1 || ld > SPEC_MAX_CONTEXT || n_min < 1 ||
      n_max < n_min || n_max > SPEC_MAX_NGRAM || K < 1 || K > SPEC_MAX_K)
    return SPEC_ERR_ARG;
  hipLaunchKernelGGL(ngram_draft_kernel, dim3(static_cast<unsigned>(B)), dim3(kLookupBlock), 0,
                     stream, context, ld, context_len, n_max, n_min, K, out_tokens, out_len,
                     out_ngram, out_src);
  return launch_status();
}
