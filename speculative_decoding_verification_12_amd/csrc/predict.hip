// Outcome-key prediction on gfx950.
//
// Method (page "Speculative Speculative Decoding (SSD)", section "1. Outcome Prediction (The
// Saguaro Cache)": the outcome of a verification is how many drafts were kept plus the token the
// target placed, and the placed token is predicted from the draft's top logits; page
// "LLMの生成を5倍速くする「D3D」を図で読む", section "答え:…": an outcome is (kept count, placed
// token)); page "LLMの生成を5倍速くする「D3D」を図で読む", sections "答え:…", "ヒット", "ミス":
// for each of the first P slots the drafter prepares candidates for the token the target would
// place there, its own top choices other than the draft token, plus one continuation for the case
// where every draft is kept). For every slot k < P the F_k tokens with the largest draft logits,
// ordered by logit descending then id ascending and optionally skipping the draft token x_k, are
// the keys (k, t); at T > 0 each key also gets q_k(t). The uniform case (F_k = F for every slot,
// no exclusion) is spec_predict_outcomes; the per-slot case is spec_predict_fanout. A second,
// tiny kernel maps each verification outcome to the prepared continuation it selects.
//
// Two launches:
//  1. predict_stats_kernel: a workgroup per (request, slot, chunk), in chunks small enough that
//     the grid runs in several rounds of workgroups (so one workgroup's arithmetic overlaps the
//     loads of others). It streams its chunk once and stores the chunk's maximum, at T > 0 its
//     sum of 2^((l - max) c), and the maxima of its four waves. No workgroup waits for
//     another: the kernel boundary is the only synchronisation.
//  2. predict_select_kernel: a workgroup of eight waves per slot merges the chunk statistics into
//     the row's (M, S) and selects the keys from the wave maxima (select_keys: only the waves
//     whose maximum reaches the F'-th largest wave maximum can hold a key, and only those are
//     read again).
// With the draft token excluded a slot looks for F_k + 1 tokens and drops x_k (or, when x_k is
// not among them, the last one).
#include "api_common.hpp"
#include "row_keys.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

// Per-slot work of one launch, passed by value: slot k < P looks for pick[k] tokens and writes
// count[k] keys at offset off[k] of its request's S keys (pick = count, or count + 1 when the
// draft token is excluded; 0 skips the slot).
struct FanoutTable {
  int P;
  int S;
  // 32-bit entries: a workgroup reads its slot's entries with a uniform runtime index, which a
  // scalar load serves only for whole dwords (a byte entry became a vector load and a wait for
  // it before the workgroup's first row load)
  int32_t pick[SPEC_MAX_K];
  int32_t count[SPEC_MAX_K];
  int32_t off[SPEC_MAX_K];
};

template <typename TIn>
__global__ __launch_bounds__(kBlock) void predict_stats_kernel(const TIn* __restrict__ drf, int K,
                                                               int V, FanoutTable ft, float c,
                                                               int nchunk, int cv,
                                                               float2* __restrict__ part,
                                                               float* __restrict__ wmax) {
  __shared__ float sm[kWaves], ss[kWaves];
  const int ch = blockIdx.x % nchunk;
  const int rk = blockIdx.x / nchunk;   // b * P + k
  const int k = rk % ft.P, b = rk / ft.P;
  if (ft.pick[k] == 0) return;   // the whole slot is skipped
  const TIn* row = drf + (static_cast<size_t>(b) * K + k) * static_cast<size_t>(V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);
  float m, s, M, S;
  // non-temporal loads: afterwards only the few waves that can hold a key are read again
  // (measured ~1 us faster per C5 call than ordinary loads)
  if (c > 0.f)
    thread_chunk_stats<TIn, true, true>(row, sp, cr, V, c, m, s);
  else
    thread_chunk_stats<TIn, false, true>(row, sp, cr, V, c, m, s);
  const size_t pc = static_cast<size_t>(rk) * nchunk + ch;
  block_stats(m, s, c, sm, ss, M, S, wmax + pc * kWaves);
  if (threadIdx.x == 0) part[pc] = make_float2(M, S);
}

// One workgroup of kSelectWaves waves per slot.
constexpr int kSelectWaves = 8;

template <typename TIn>
__global__ __launch_bounds__(kSelectWaves * kWave) void predict_select_kernel(
    const TIn* __restrict__ drf, const int32_t* __restrict__ xtok, int K, int V, FanoutTable ft,
    float c, int nchunk, int cv, const float2* __restrict__ part, const float* __restrict__ wmax,
    int32_t* __restrict__ out_keys, float* __restrict__ out_prob) {
  const int rk = blockIdx.x;   // b * P + k
  const int k = rk % ft.P, b = rk / ft.P;
  const int Fp = ft.pick[k];
  if (Fp == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int xk = xtok ? xtok[static_cast<size_t>(b) * K + k] : -1;   // excluded token, if any
  // the chunk statistics, loaded now and merged by wave 0 only when the keys are written
  const float2* pr = part + static_cast<size_t>(rk) * nchunk;
  // (every lane loads, from a clamped index, so no wait for it comes before the maxima's loads)
  const float2 a0r = load_f2(pr + min(lane, nchunk - 1));
  auto row_stat = [&]() {   // the row's (M, S) from its chunks (wave 0)
    const float2 a0 = lane < nchunk ? a0r : make_float2(-INFINITY, 0.f);
    float lm = a0.x;
    for (int j = lane + kWave; j < nchunk; j += kWave) lm = fmaxf(lm, load_f2(pr + j).x);
    const float Mr = wave_max(lm);
    double ls = 0.0;
    if (c > 0.f) {
      if (a0.x > -INFINITY) ls += static_cast<double>(a0.y) * rel_exp2(a0.x, Mr, c);
      for (int j = lane + kWave; j < nchunk; j += kWave) {
        const float2 a = load_f2(pr + j);
        if (a.x > -INFINITY) ls += static_cast<double>(a.y) * rel_exp2(a.x, Mr, c);
      }
    }
    return RowStat{Mr, 0.f, wave_sum(ls)};
  };
  const size_t o = static_cast<size_t>(b) * ft.S + ft.off[k];
  select_keys<TIn, kSelectWaves, false>(
      drf + (static_cast<size_t>(b) * K + k) * static_cast<size_t>(V), V, nchunk, cv,
      wmax + static_cast<size_t>(rk) * nchunk * kWaves, Fp, ft.count[k], xk, row_stat, c,
      out_keys + o, out_prob ? out_prob + o : nullptr);
}

template <typename TIn>
int launch_predict(const void* draft, const int32_t* xtok, int B, int K, int V,
                   const FanoutTable& ft, float T, int32_t* out_keys, float* out_prob, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  // chunking as for all K slots of every request, so the workspace sized by
  // spec_workspace_bytes(B, K, V, .) covers any P <= K
  const KernelPlan P = predict_plan(B, K, V, 16 / static_cast<int>(sizeof(TIn)));
  const size_t g = static_cast<size_t>(B) * ft.P * P.nchunk;
  if (!grid_fits(g)) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1, ws_bytes);
  const float c = T > 0.f ? exp2_scale(T) : 0.f;
  float2* part = ws_ptr<float2>(ws, L.part_pred);
  float* wm = ws_ptr<float>(ws, L.part_pwm);
  const TIn* d = static_cast<const TIn*>(draft);
  hipLaunchKernelGGL(predict_stats_kernel<TIn>, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0,
                     stream, d, K, V, ft, c, P.nchunk, P.cv, part, wm);
  hipLaunchKernelGGL(predict_select_kernel<TIn>, dim3(static_cast<unsigned>(B) * ft.P),
                     dim3(kSelectWaves * kWave), 0, stream, d, xtok, K, V, ft, c, P.nchunk, P.cv,
                     static_cast<const float2*>(part), static_cast<const float*>(wm), out_keys,
                     out_prob);
  return launch_status();
}

int check_predict_common(const void* draft_logits, int dtype, int B, int K, int V,
                         float temperature, const int32_t* out_keys) {
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (check_logits(draft_logits, dtype) != SPEC_OK || out_keys == nullptr) return SPEC_ERR_ARG;
  if (!std::isfinite(temperature) || temperature < 0.f ||
      (temperature > 0.f && !std::isfinite(exp2_scale(temperature))))
    return SPEC_ERR_TEMPERATURE;
  return SPEC_OK;
}

int run_predict(const void* draft_logits, int dtype, const int32_t* xtok, int B, int K, int V,
                const FanoutTable& ft, float temperature, int32_t* out_keys, float* out_key_prob,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return launch_predict<uint16_t>(draft_logits, xtok, B, K, V, ft, temperature, out_keys,
                                    out_key_prob, workspace, workspace_bytes, stream);
  return launch_predict<float>(draft_logits, xtok, B, K, V, ft, temperature, out_keys,
                               out_key_prob, workspace, workspace_bytes, stream);
}

// Builds the per-slot table; false when a fan-out is out of range.
bool fanout_table(const int32_t* fanout, int P, bool exclude, int V, FanoutTable& ft) {
  ft.P = P;
  ft.S = 0;
  for (int k = 0; k < SPEC_MAX_K; ++k) {
    ft.pick[k] = 0;
    ft.count[k] = 0;
    ft.off[k] = 0;
  }
  for (int k = 0; k < P; ++k) {
    const int F = fanout[k];
    const int pick = F > 0 ? F + (exclude ? 1 : 0) : 0;
    if (F < 0 || pick > SPEC_MAX_F || pick > V) return false;
    ft.pick[k] = pick;
    ft.count[k] = F;
    ft.off[k] = ft.S;
    ft.S += F;
  }
  return ft.S > 0;
}

// ------------------------------------------------------------------------------ lookup
// One thread per request: the outcome (tau, placed token) against the request's keys.
__global__ __launch_bounds__(kBlock) void lookup_kernel(const int32_t* __restrict__ tau,
                                                        const int32_t* __restrict__ tokens,
                                                        const int32_t* __restrict__ keys, int B,
                                                        int K, FanoutTable ft, int all_accept,
                                                        int32_t* __restrict__ out_slot) {
  const int b = blockIdx.x * kBlock + threadIdx.x;
  if (b >= B) return;
  const int tb = tau[b];
  int slot = -1;
  if (tb == K + 1) {
    slot = all_accept ? ft.S : -1;
  } else if (tb >= 1 && tb <= K && tb - 1 < ft.P) {
    const int m = tb - 1;
    const int y = tokens[static_cast<size_t>(b) * (K + 1) + m];
    const int32_t* kr = keys + static_cast<size_t>(b) * ft.S + ft.off[m];
    for (int j = 0; j < ft.count[m]; ++j)
      if (kr[j] == y) {
        slot = ft.off[m] + j;
        break;
      }
  }
  out_slot[b] = slot;
}

}  // namespace
}  // namespace sv

extern "C" int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int K, int V,
                                     int F, float temperature, int32_t* out_keys,
                                     float* out_key_prob, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  using namespace sv;
  int rc = check_predict_common(draft_logits, dtype, B, K, V, temperature, out_keys);
  if (rc != SPEC_OK) return rc;
  if (F < 1 || F > SPEC_MAX_F || F > V) return SPEC_ERR_ARG;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, F)) != SPEC_OK) return rc;
  int32_t fan[SPEC_MAX_K];
  for (int k = 0; k < K; ++k) fan[k] = F;
  FanoutTable ft;
  if (!fanout_table(fan, K, false, V, ft)) return SPEC_ERR_ARG;
  return run_predict(draft_logits, dtype, nullptr, B, K, V, ft, temperature, out_keys,
                     out_key_prob, workspace, workspace_bytes, stream);
}

extern "C" int spec_predict_fanout(const void* draft_logits, int dtype,
                                   const int32_t* draft_tokens, int B, int K, int V, int P,
                                   const int32_t* fanout, float temperature, int32_t* out_keys,
                                   float* out_key_prob, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  using namespace sv;
  int rc = check_predict_common(draft_logits, dtype, B, K, V, temperature, out_keys);
  if (rc != SPEC_OK) return rc;
  if (P < 1 || P > K || fanout == nullptr) return SPEC_ERR_ARG;
  FanoutTable ft;
  if (!fanout_table(fanout, P, draft_tokens != nullptr, V, ft)) return SPEC_ERR_ARG;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, 1)) != SPEC_OK) return rc;
  return run_predict(draft_logits, dtype, draft_tokens, B, K, V, ft, temperature, out_keys,
                     out_key_prob, workspace, workspace_bytes, stream);
}

extern "C" int spec_outcome_lookup(const int32_t* tau, const int32_t* tokens,
                                   const int32_t* keys, int B, int K, int P,
                                   const int32_t* fanout, int all_accept, int32_t* out_slot,
                                   hipStream_t stream) {
  using namespace sv;
  if (tau == nullptr || tokens == nullptr || keys == nullptr || out_slot == nullptr ||
      fanout == nullptr || B < 1 || K < 1 || K > SPEC_MAX_K || P < 1 || P > K)
    return SPEC_ERR_ARG;
  FanoutTable ft;
  // the key lists only need count/off here; V does not constrain a lookup
  if (!fanout_table(fanout, P, false, SPEC_MAX_V, ft)) return SPEC_ERR_ARG;
  const unsigned blocks = static_cast<unsigned>((B + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(lookup_kernel, dim3(blocks), dim3(kBlock), 0, stream, tau, tokens, keys, B,
                     K, ft, all_accept ? 1 : 0, out_slot);
  return launch_status();
}
