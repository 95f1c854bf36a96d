// Paged KV-cache rewind after verification (page "speculative decodingとは", section
// "speculative decodingとKV cache、プロンプトキャッシュの関係は?": both models append the drafts'
// keys and values to their caches, and when the target rejects the drafts after position m the
// engine truncates both caches, dropping the rejected entries, before the next round).
//
// Request b's entries [0, L) live in blocks table[b][0 .. ceil(L / bs)). Keeping L' of L entries
// releases the whole blocks [ceil(L' / bs), ceil(L / bs)); their table entries become -1 and their
// ids are listed request by request (in table order within a request), at offsets given by an
// exclusive prefix sum of the per-request counts, so the list is the same on every run. One
// workgroup walks the batch in tiles of 256 requests, one thread per request, with a block
// prefix scan per tile; the work is a few integer operations per request.
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

__global__ __launch_bounds__(kBlock) void kv_rewind_kernel(int32_t* __restrict__ tables, int B,
                                                           int max_blocks, int bs,
                                                           const int32_t* __restrict__ kv_alloc,
                                                           const int32_t* __restrict__ kv_new,
                                                           int32_t* __restrict__ out_freed,
                                                           int32_t* __restrict__ out_offsets) {
  __shared__ int s_wave[kWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int running = 0;   // uniform: ids listed by earlier tiles
  for (int base = 0; base < B; base += kBlock) {
    const int b = base + tid;
    int held = 0, kept = 0;
    if (b < B) {
      const long long la = kv_alloc[b] > 0 ? kv_alloc[b] : 0;
      const long long ln = kv_new[b] > 0 ? kv_new[b] : 0;
      held = static_cast<int>(min(static_cast<long long>(max_blocks), (la + bs - 1) / bs));
      kept = static_cast<int>(min(static_cast<long long>(max_blocks), (ln + bs - 1) / bs));
    }
    const int cnt = held > kept ? held - kept : 0;
    const int incl = wave_scan_incl(cnt);
    if (lane == kWave - 1) s_wave[w] = incl;
    __syncthreads();
    int off = running, tile = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      if (i < w) off += s_wave[i];
      tile += s_wave[i];
    }
    off += incl - cnt;
    if (b < B) {
      int32_t* row = tables + static_cast<size_t>(b) * max_blocks;
      for (int j = 0; j < cnt; ++j) {
        out_freed[off + j] = row[kept + j];
        row[kept + j] = -1;
      }
      out_offsets[b] = off;
    }
    running += tile;
    __syncthreads();   // s_wave is rewritten by the next tile
  }
  if (tid == 0) out_offsets[B] = running;
}

}  // namespace
}  // namespace sv

extern "C" int spec_kv_rewind(int32_t* block_tables, int B, int max_blocks, int block_size,
                              const int32_t* kv_alloc, const int32_t* kv_new,
                              int32_t* out_freed, int32_t* out_offsets, hipStream_t stream) {
  using namespace sv;
  if (block_tables == nullptr || kv_alloc == nullptr || kv_new == nullptr ||
      out_freed == nullptr || out_offsets == nullptr || B < 1 || max_blocks < 1 ||
      block_size < 1 || static_cast<long long>(B) * max_blocks > 0x7fffffffll)
    return SPEC_ERR_ARG;
  hipLaunchKernelGGL(kv_rewind_kernel, dim3(1), dim3(kBlock), 0, stream, block_tables, B,
                     max_blocks, block_size, kv_alloc, kv_new, out_freed, out_offsets);
  return launch_status();
}
