// Greedy verification (temperature zero) on gfx950.
//
// Method (page "speculative decodingとは", stage 3 of the four-stage loop at temperature zero;
// page "LLMの生成を5倍速くする「D3D」を図で読む", sections 検証のしくみ③ and 検証のまとめ): draft
// k is kept while it equals the target's top choice g_k for its slot; at the first mismatch m
// the target's own g_m is placed and the rest dropped; if all K match, g_K (the extra row) is
// appended. tau = m + 1, the KV length advances by tau. Ties in the target's top choice go to
// the lowest token id. Only the K+1 target rows are read; the draft logits are not needed.
// With draft lengths (drafts that carry no distribution, e.g. prompt lookup) only the first n_b
// slots hold drafts: rows past n_b are not read, and with all n_b kept the top choice of row
// n_b is appended.
//
// One launch: a workgroup per (request, row, chunk) streams its chunk once, tracks the largest
// logit and its lowest id per thread, reduces (value desc, id asc) across the workgroup and
// publishes the result as a self-flagged word in the part of the workspace that is zero between
// calls; it waits for nothing. The grid ends with one deciding workgroup per request: it polls
// the request's words, merges each row's chunks, clears the words, compares g_k with x_k in one
// wave (lane k = slot k, ballot for the first mismatch) and writes the outputs. The deciders are
// the last workgroups of the grid, so every streaming workgroup has been dispatched before they
// start, and those never wait: the polls end. They are still bounded: a decider that runs out of
// polls on a word swaps a sentinel into it (or takes the word, if it landed meanwhile), streams
// its request's rows itself (the same maxima and lowest ids), and then waits for each word it
// gave up on (its workgroup was dispatched before the decider, so it comes) and clears it: the
// workspace is left as clean as after any other call, and the next call takes the fast path.
// Only if that second wait runs out too does the decider mark the workspace; while the mark is
// set (until spec_workspace_init) every decider streams its own rows and trusts no word.
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

// The (max, lowest id) of chunk `ch` of row `rb`; the result is valid in thread 0. A caller that
// runs it again first passes a barrier (s_v, s_i are reused).
template <typename TIn>
__device__ __forceinline__ void greedy_chunk(const TIn* __restrict__ tgt, int rb, int ch, int V,
                                             int nchunk, int cv, float* s_v, int* s_i, float& M,
                                             int& I) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const TIn* row = tgt + static_cast<size_t>(rb) * static_cast<size_t>(V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);

  // Each thread visits its elements in increasing token order and keeps the first maximum.
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (cr.first && tid < sp.head) {
    const float v = E::one(row, tid);
    if (v > bv) {
      bv = v;
      bi = tid;
    }
  }
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
  for (int base = cr.vbeg; base < cr.vend; base += kPassVecs) {
    // Every lane loads, a lane past the chunk its last vector again (dropped below), so the
    // loads leave back to back with no branch between them and all are in flight at once.
    const unsigned last = static_cast<unsigned>(cr.vend - 1);
    uint4 q[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i)
      q[i] = load_stream(vrow, min(static_cast<unsigned>(base + i * kBlock + tid), last));
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i)
      if (static_cast<unsigned>(base + i * kBlock + tid) > last) q[i] = neg_inf_vec<TIn>();
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      float t[N];
      E::unpack(q[i], t);
      const int tok0 = sp.head + (base + i * kBlock + tid) * N;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        if (t[j] > bv) {
          bv = t[j];
          bi = tok0 + j;
        }
      }
    }
  }
  if (cr.last && tid < V - sp.tail) {
    const float v = E::one(row, sp.tail + tid);
    if (v > bv) {
      bv = v;
      bi = sp.tail + tid;
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    M = s_v[0];
    I = s_i[0];
    for (int k = 1; k < kWaves; ++k)
      if (better(s_v[k], s_i[k], M, I)) {
        M = s_v[k];
        I = s_i[k];
      }
  }
}

// Published word of a chunk: (max, lowest id) with bit 31 of the id set as the written flag
// (ids are below 2^31; an all -inf chunk keeps the id 0x7fffffff).
constexpr uint64_t kArgFlag = 1ull << 63;
// What a decider leaves in a word it stopped waiting for (never a published word: no flag).
constexpr uint64_t kAbandoned = 1ull;

template <typename TIn>
__global__ __launch_bounds__(kBlock) void greedy_kernel(
    const TIn* __restrict__ tgt, const int32_t* __restrict__ xtok,
    const int32_t* __restrict__ kv_in, int K, int V, int nchunk, int cv, int nstream,
    uint64_t* __restrict__ words, unsigned* __restrict__ mark, int wait_polls,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_tau, int32_t* __restrict__ out_kv,
    const int32_t* __restrict__ dlen, float* __restrict__ out_p, float* __restrict__ out_q) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ int row_g[SPEC_MAX_K + 1];
  __shared__ int s_late;

  const int rows = K + 1;
  const bool decider = static_cast<int>(blockIdx.x) >= nstream;
  const int rb = decider ? 0 : static_cast<int>(blockIdx.x) / nchunk;   // b * (K+1) + row
  const int b = decider ? static_cast<int>(blockIdx.x) - nstream : rb / rows;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  // drafts in this request: K, or the first dlen[b] slots (outside [0, K]: a row error)
  int nb = K;
  bool nb_bad = false;
  if (dlen != nullptr) {
    nb = dlen[b];
    nb_bad = nb < 0 || nb > K;
    if (nb_bad) nb = -1;
  }

  if (!decider) {
    // a row past n_b is never used by an outcome: it is not read and publishes nothing
    if (rb % rows > nb) return;
    const int ch = static_cast<int>(blockIdx.x) % nchunk;
    float M;
    int I;
    greedy_chunk<TIn>(tgt, rb, ch, V, nchunk, cv, s_v, s_i, M, I);
    if (tid == 0)
      store_coherent(words + static_cast<size_t>(rb) * nchunk + ch, pack2(M, I) | kArgFlag);
    return;
  }

  // ---- decider of request b: per-row argmax over the published chunks (rows up to n_b), each
  // row by a group of lanes, every word polled at once; it clears each word it has read. Every call's chunk
  // workgroups publish their words, so the polls end whether or not the mark is set; the mark,
  // read alongside them, only decides afterwards whether the words are trusted.
  // wave 0's decision inputs (lane k: draft token k; the KV length) are loaded first, so their
  // latency passes while the words are polled
  const int k = lane;
  const bool valid = k < nb;
  const int xk = (w == 0 && valid) ? xtok[static_cast<size_t>(b) * K + k] : 0;
  const int kv0 = (w == 0 && kv_in != nullptr) ? kv_in[b] : 0;
  if (tid == 0) s_late = 0;
  __syncthreads();
  const bool marked = load_coherent_u32(mark) != 0u;
  bool late = false;
  // rows in groups of G lanes (G = nchunk rounded up to a power of two, at most a wave), so the
  // block polls every word of up to 4 * 64 / G rows at once
  int G = 1;
  while (G < nchunk && G < kWave) G <<= 1;
  const int per_wave = kWave / G, g = lane / G, gi = lane % G;
  const int nrows = min(rows, nb + 1);   // rows 0..n_b (none for a bad length)
  for (int base = 0; base < nrows; base += kWaves * per_wave) {
    const int rr = base + w * per_wave + g;
    float v = -INFINITY;
    int i = 0x7fffffff;
    if (rr < nrows) {
      uint64_t* pw = words + (static_cast<size_t>(b) * rows + rr) * nchunk;
      for (int j = gi; j < nchunk; j += G) {
        uint64_t a = load_coherent(pw + j);
        for (int polls = wait_polls; (a & kArgFlag) == 0ull && polls > 0; --polls) {
          __builtin_amdgcn_s_sleep(2);
          a = load_coherent(pw + j);
        }
        if ((a & kArgFlag) == 0ull) {
          // give up on this word: the sentinel tells the clean-up below that its publish is
          // still to come; a publish that lands first makes the swap fail and is taken here
          a = cas_coherent(pw + j, 0ull, kAbandoned);
          if ((a & kArgFlag) == 0ull) {
            late = true;
            continue;
          }
        }
        a &= ~kArgFlag;
        if (better(lo_float(a), hi_int(a), v, i)) {
          v = lo_float(a);
          i = hi_int(a);
        }
        store_coherent(pw + j, 0ull);   // read: back to zero for the next call
      }
    }
    // the group's (max, lowest id): the same pair whatever the order of the merges
    for (int off = G / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off, kWave);
      const int oi = __shfl_xor(i, off, kWave);
      if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    if (gi == 0 && rr < nrows) row_g[rr] = (i == 0x7fffffff) ? 0 : i;   // all -inf: lowest id
  }
  if (__any(late || marked) && lane == 0) s_late = 1;
  __syncthreads();
  if (s_late != 0) {
    // a row's words did not all arrive within the poll budget, or the mark was set: stream the
    // request's rows here, chunk by chunk in order (so the same maximum and lowest id)
    for (int rr = 0; rr < rows && rr <= nb; ++rr) {
      float v = -INFINITY;
      int i = 0x7fffffff;
      for (int ch = 0; ch < nchunk; ++ch) {
        float M;
        int I;
        greedy_chunk<TIn>(tgt, b * rows + rr, ch, V, nchunk, cv, s_v, s_i, M, I);
        if (tid == 0 && better(M, I, v, i)) {
          v = M;
          i = I;
        }
        __syncthreads();   // s_v, s_i are reused
      }
      if (tid == 0) row_g[rr] = (i == 0x7fffffff) ? 0 : i;
    }
    // clean-up: every word of the request given up on above is published by now or soon (its
    // workgroup was dispatched before this one); wait for it and clear it, and clear any word
    // that landed after the polls, so the request's words are all zero again for the next call.
    // A word still not there after a full budget marks the workspace.
    bool stuck = false;
    for (int rr = w; rr < rows && rr <= nb; rr += kWaves) {
      uint64_t* pw = words + (static_cast<size_t>(b) * rows + rr) * nchunk;
      for (int j = lane; j < nchunk; j += kWave) {
        uint64_t a = load_coherent(pw + j);
        for (int polls = SPEC_DEFAULT_WAIT_POLLS; a == kAbandoned && polls > 0; --polls) {
          __builtin_amdgcn_s_sleep(2);
          a = load_coherent(pw + j);
        }
        if (a == kAbandoned) stuck = true;
        else if (a != 0ull) store_coherent(pw + j, 0ull);
      }
    }
    if (__syncthreads_or(stuck) && tid == 0) store_coherent_u32(mark, 1u);
    __syncthreads();
  }
  if (w != 0) return;

  const bool bad = valid && (xk < 0 || xk >= V);
  const bool err = nb_bad || __ballot(bad) != 0ull;
  const unsigned long long miss = __ballot(valid && xk != row_g[valid ? k : 0]);
  const int mm = err ? 0 : (miss ? (__ffsll(static_cast<long long>(miss)) - 1) : nb);
  if (out_p != nullptr && k < K) {   // at temperature zero: p_k(x_k) is the top-choice indicator
    const size_t o = static_cast<size_t>(b) * K + k;
    out_p[o] = (err || !valid) ? NAN : (xk == row_g[k] ? 1.f : 0.f);
    if (out_q) out_q[o] = (err || !valid) ? NAN : 1.f;
  }
  for (int j = lane; j <= K; j += kWave) {
    int tok = -1;
    if (!err) tok = j < mm ? xk : (j == mm ? row_g[mm] : -1);
    out_tok[static_cast<size_t>(b) * (K + 1) + j] = tok;
  }
  if (lane == 0) {
    out_tau[b] = err ? -1 : mm + 1;
    if (out_kv) out_kv[b] = err ? kv0 : kv0 + mm + 1;
  }
}

template <typename TIn>
int launch_greedy(const void* target, const int32_t* xtok, const int32_t* kv_in, int B, int K,
                  int V, int32_t* out_tok, int32_t* out_tau, int32_t* out_kv, void* ws,
                  size_t ws_bytes, hipStream_t stream, int wait_polls,
                  const int32_t* dlen = nullptr, float* out_p = nullptr,
                  float* out_q = nullptr) {
  const KernelPlan P = greedy_plan(B, K, V, 16 / static_cast<int>(sizeof(TIn)));
  const size_t nstream = static_cast<size_t>(B) * (K + 1) * P.nchunk;
  const size_t g = nstream + static_cast<size_t>(B);   // the deciders come last
  if (!grid_fits(g)) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1, ws_bytes);
  hipLaunchKernelGGL(greedy_kernel<TIn>, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0, stream,
                     static_cast<const TIn*>(target), xtok, kv_in, K, V, P.nchunk, P.cv,
                     static_cast<int>(nstream), ws_ptr<uint64_t>(ws, L.greedy_words),
                     ws_ptr<unsigned>(ws, L.greedy_mark),
                     wait_polls < 0 ? SPEC_DEFAULT_WAIT_POLLS : wait_polls, out_tok, out_tau,
                     out_kv, dlen, out_p, out_q);
  return launch_status();
}

}  // namespace

int greedy_point_entry(const void* target, int dtype, const int32_t* xtok, const int32_t* dlen,
                       const int32_t* kv_in, int B, int K, int V, int32_t* out_tok,
                       int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return launch_greedy<uint16_t>(target, xtok, kv_in, B, K, V, out_tok, out_tau, out_kv, ws,
                                   ws_bytes, stream, -1, dlen, out_p, out_q);
  return launch_greedy<float>(target, xtok, kv_in, B, K, V, out_tok, out_tau, out_kv, ws,
                              ws_bytes, stream, -1, dlen, out_p, out_q);
}
}  // namespace sv

extern "C" int spec_verify_greedy_ex(const void* target_logits, int dtype,
                                     const int32_t* draft_tokens, const int32_t* kv_len_in, int B,
                                     int K, int V, float temperature, int32_t* out_tokens,
                                     int32_t* out_tau, int32_t* out_kv_len, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream, int wait_polls) {
  using namespace sv;
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (check_logits(target_logits, dtype) != SPEC_OK || draft_tokens == nullptr ||
      out_tokens == nullptr || out_tau == nullptr)
    return SPEC_ERR_ARG;
  if (temperature != 0.f) return SPEC_ERR_TEMPERATURE;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, 1)) != SPEC_OK) return rc;
  if (dtype == SPEC_BF16)
    return launch_greedy<uint16_t>(target_logits, draft_tokens, kv_len_in, B, K, V, out_tokens,
                                   out_tau, out_kv_len, workspace, workspace_bytes, stream,
                                   wait_polls);
  return launch_greedy<float>(target_logits, draft_tokens, kv_len_in, B, K, V, out_tokens,
                              out_tau, out_kv_len, workspace, workspace_bytes, stream, wait_polls);
}

extern "C" int spec_verify_greedy(const void* target_logits, int dtype,
                                  const int32_t* draft_tokens, const int32_t* kv_len_in, int B,
                                  int K, int V, float temperature, int32_t* out_tokens,
                                  int32_t* out_tau, int32_t* out_kv_len, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return spec_verify_greedy_ex(target_logits, dtype, draft_tokens, kv_len_in, B, K, V,
                               temperature, out_tokens, out_tau, out_kv_len, workspace,
                               workspace_bytes, stream, -1);
}
