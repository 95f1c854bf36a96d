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
// logit and its lowest id per thread, and reduces (value desc, id asc) across the workgroup. The
// request's last workgroup to arrive merges the chunks, compares g_k with x_k in one wave
// (lane k = slot k, ballot for the first mismatch) and writes the outputs.
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

// The (max, lowest id) of chunk `ch` of row `rb`, stored as that chunk's partial.
template <typename TIn>
__device__ __forceinline__ void greedy_chunk(const TIn* __restrict__ tgt, int rb, int ch, int V,
                                             int nchunk, int cv, ArgPart* __restrict__ part,
                                             float* s_v, int* s_i) {
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
    uint4 q[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int vi = base + i * kBlock + tid;
      q[i] = vi < cr.vend ? load_stream(vrow, vi) : neg_inf_vec<TIn>();
    }
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
    float v = s_v[0];
    int i = s_i[0];
    for (int k = 1; k < kWaves; ++k)
      if (better(s_v[k], s_i[k], v, i)) {
        v = s_v[k];
        i = s_i[k];
      }
    store_coherent(&part[static_cast<size_t>(rb) * nchunk + ch], pack2(v, i));
  }
}

template <typename TIn>
__global__ __launch_bounds__(kBlock) void greedy_kernel(
    const TIn* __restrict__ tgt, const int32_t* __restrict__ xtok,
    const int32_t* __restrict__ kv_in, int K, int V, int nchunk, int cv,
    ArgPart* __restrict__ part, unsigned* __restrict__ cnt_base, int32_t* __restrict__ out_tok,
    int32_t* __restrict__ out_tau, int32_t* __restrict__ out_kv,
    const int32_t* __restrict__ dlen, float* __restrict__ out_p, float* __restrict__ out_q) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ int s_flag;
  __shared__ int row_g[SPEC_MAX_K + 1];

  const int rows = K + 1;
  const int ch = blockIdx.x % nchunk;
  const int rb = blockIdx.x / nchunk;   // b * (K+1) + row
  const int b = rb / rows;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  unsigned* cnt = cnt_base + static_cast<size_t>(b) * kCounterStride;
  // drafts in this request: K, or the first dlen[b] slots (outside [0, K]: a row error)
  int nb = K;
  bool nb_bad = false;
  if (dlen != nullptr) {
    nb = dlen[b];
    nb_bad = nb < 0 || nb > K;
    if (nb_bad) nb = -1;
  }
  // a row past n_b is never used by an outcome: it is not read, but its workgroups still arrive
  if (rb % rows <= nb) greedy_chunk<TIn>(tgt, rb, ch, V, nchunk, cv, part, s_v, s_i);
  if (!arrive_last(cnt, static_cast<unsigned>(rows * nchunk), &s_flag)) return;

  // ---- last workgroup of request b: per-row argmax over chunks (rows up to n_b)
  for (int rr = w; rr < rows && rr <= nb; rr += kWaves) {
    const ArgPart* pr = part + (static_cast<size_t>(b) * rows + rr) * nchunk;
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int j = lane; j < nchunk; j += kWave) {
      const uint64_t a = load_coherent(&pr[j]);
      if (better(lo_float(a), hi_int(a), v, i)) {
        v = lo_float(a);
        i = hi_int(a);
      }
    }
    wave_argmax(v, i);
    // a row whose logits are all -inf keeps no index: its first token is the lowest id
    if (lane == 0) row_g[rr] = (i == 0x7fffffff) ? 0 : i;
  }
  __syncthreads();
  if (w != 0) return;

  const int k = lane;
  const bool valid = k < nb;
  const int xk = valid ? xtok[static_cast<size_t>(b) * K + k] : 0;
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
    const int kv0 = kv_in ? kv_in[b] : 0;
    out_tau[b] = err ? -1 : mm + 1;
    if (out_kv) out_kv[b] = err ? kv0 : kv0 + mm + 1;
    reset_counter(cnt);
  }
}

template <typename TIn>
int launch_greedy(const void* target, const int32_t* xtok, const int32_t* kv_in, int B, int K,
                  int V, int32_t* out_tok, int32_t* out_tau, int32_t* out_kv, void* ws,
                  size_t ws_bytes, hipStream_t stream, const KernelPlan& P,
                  const int32_t* dlen = nullptr,
                  float* out_p = nullptr, float* out_q = nullptr) {
  const size_t g = static_cast<size_t>(B) * (K + 1) * P.nchunk;
  if (!grid_fits(g)) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1, ws_bytes);
  hipLaunchKernelGGL(greedy_kernel<TIn>, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0, stream,
                     static_cast<const TIn*>(target), xtok, kv_in, K, V, P.nchunk, P.cv,
                     ws_ptr<ArgPart>(ws, L.part_greedy), ws_ptr<unsigned>(ws, L.cnt_a), out_tok,
                     out_tau, out_kv, dlen, out_p, out_q);
  return launch_status();
}

}  // namespace

int greedy_point_entry(const void* target, int dtype, const int32_t* xtok, const int32_t* dlen,
                       const int32_t* kv_in, int B, int K, int V, int32_t* out_tok,
                       int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return launch_greedy<uint16_t>(target, xtok, kv_in, B, K, V, out_tok, out_tau, out_kv, ws,
                                   ws_bytes, stream, greedy_plan(B, K, V, 8), dlen, out_p, out_q);
  return launch_greedy<float>(target, xtok, kv_in, B, K, V, out_tok, out_tau, out_kv, ws,
                              ws_bytes, stream, greedy_plan(B, K, V, 4), dlen, out_p, out_q);
}
}  // namespace sv

extern "C" int spec_verify_greedy(const void* target_logits, int dtype,
                                  const int32_t* draft_tokens, const int32_t* kv_len_in, int B,
                                  int K, int V, float temperature, int32_t* out_tokens,
                                  int32_t* out_tau, int32_t* out_kv_len, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
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
                                   greedy_plan(B, K, V, 8));
  return launch_greedy<float>(target_logits, draft_tokens, kv_len_in, B, K, V, out_tokens,
                              out_tau, out_kv_len, workspace, workspace_bytes, stream,
                              greedy_plan(B, K, V, 4));
}
