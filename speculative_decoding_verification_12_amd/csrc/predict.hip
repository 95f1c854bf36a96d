// Outcome-key prediction on gfx950.
//
// Method (page "Speculative Speculative Decoding (SSD)", section "1. Outcome Prediction (The
// Saguaro Cache)": the outcome of a verification is how many drafts were kept plus the token the
// target placed, and the placed token is predicted from the draft's top logits; page
// "LLMの生成を5倍速くする「D3D」を図で読む", section "答え:…": an outcome is (kept count, placed
// token)). For every draft slot k the F tokens with the largest draft logits, ordered by logit
// descending then id ascending, are the keys (k, t); at T > 0 each key also gets q_k(t).
//
// One launch: a workgroup per (request, slot, chunk of at most 1024 16-byte vectors). Each thread holds
// its 8..34 elements in registers for one pass. Exact top-F of the chunk without sorting it:
//   1. every wave picks its F largest lane maxima; theta = the largest of the waves' F-th values.
//      Some wave then holds F elements >= theta, so every element of the chunk's top F is
//      >= theta and lives in a lane whose maximum is >= theta;
//   2. only those candidate lanes (a handful) copy their elements to LDS;
//   3. one wave selects the top F among the candidates by F rounds of (value, id) argmax, each
//      round excluding everything at or before the previous pick in that order.
// At T > 0 the same pass also keeps the online (max, scaled sum) for the key probabilities. The
// slot's last workgroup to arrive merges the chunks' lists and statistics.
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

constexpr int kCandSlots = 16;   // candidate lanes copied to LDS per batch
constexpr int kSentinelId = 0x7fffffff;

// after (pv, pi) in the order (value desc, id asc)
__device__ __forceinline__ bool after(float v, int i, float pv, int pi) {
  return v < pv || (v == pv && i > pi);
}

template <int n>
__device__ __forceinline__ void absorb_stats(const float (&v)[n], float c, float& m, float& s) {
  float bm = v[0];
#pragma unroll
  for (int j = 1; j < n; ++j) bm = fmaxf(bm, v[j]);
  if (bm > m) {
    s *= fast_exp2(m * c - bm * c);
    m = bm;
  }
  if (m > -INFINITY) {
    const float mc = m * c;
#pragma unroll
    for (int j = 0; j < n; ++j) s += fast_exp2(fmaf(v[j], c, -mc));
  }
}

template <typename TIn>
__global__ __launch_bounds__(kBlock) void predict_kernel(
    const TIn* __restrict__ drf, int K, int V, int F, float c, int nchunk, int cv,
    ArgPart* __restrict__ part, float2* __restrict__ pstat, unsigned* __restrict__ cnt_base,
    int32_t* __restrict__ out_keys, float* __restrict__ out_prob) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  constexpr int kPer = kVecPerThread * N + 2;                         // elements a lane holds
  constexpr int kSel = (kCandSlots * kPer + kWave - 1) / kWave;       // per selecting lane
  __shared__ uint4 c_vec[kCandSlots][kVecPerThread];
  __shared__ float c_ext[kCandSlots][2];
  __shared__ int c_tid[kCandSlots];
  __shared__ float l_v[SPEC_MAX_F];
  __shared__ int l_i[SPEC_MAX_F];
  __shared__ float s_theta[kWaves];
  __shared__ int s_cnt[kWaves];
  __shared__ float sm[kWaves], ss[kWaves];
  __shared__ int s_flag;

  const int ch = blockIdx.x % nchunk;
  const int rk = blockIdx.x / nchunk;   // b * K + k
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  unsigned* cnt = cnt_base + static_cast<size_t>(rk) * kCounterStride;
  const TIn* row = drf + static_cast<size_t>(rk) * static_cast<size_t>(V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);   // cv <= one pass (kPassVecs)

  // ---- load the lane's elements (one pass; padding is -inf)
  uint4 q[kVecPerThread];
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int vi = cr.vbeg + i * kBlock + tid;
    q[i] = vi < cr.vend ? vrow[vi] : neg_inf_vec<TIn>();
  }
  const bool has_head = cr.first && tid < sp.head;
  const bool has_tail = cr.last && tid < V - sp.tail;
  float ext[2];
  ext[0] = has_head ? E::one(row, tid) : -INFINITY;
  ext[1] = has_tail ? E::one(row, sp.tail + tid) : -INFINITY;
  const bool has = has_head || has_tail || (cr.vbeg + tid < cr.vend);

  float v[kVecPerThread * N];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    float t[N];
    E::unpack(q[i], t);
#pragma unroll
    for (int j = 0; j < N; ++j) v[i * N + j] = t[j];
  }
  float tm = fmaxf(ext[0], ext[1]);
#pragma unroll
  for (int j = 0; j < kVecPerThread * N; ++j) tm = fmaxf(tm, v[j]);

  // ---- statistics for q_k(key) at T > 0
  float M = -INFINITY, S = 0.f;
  if (c > 0.f) {
    float m = -INFINITY, s = 0.f;
    absorb_stats(ext, c, m, s);
    absorb_stats(v, c, m, s);
    const float wm = wave_max(m);
    const float sc = (m > -INFINITY) ? s * fast_exp2(m * c - wm * c) : 0.f;
    const float wsum = wave_sum(sc);
    if (lane == 0) {
      sm[w] = wm;
      ss[w] = wsum;
    }
  }

  // ---- theta: each wave's F-th largest lane maximum (lanes without elements never count)
  {
    float kv = has ? tm : -INFINITY;
    int ki = has ? lane : kSentinelId;
    float th = -INFINITY;
    int thi = kSentinelId;
    for (int f = 0; f < F; ++f) {
      float bv = kv;
      int bi = ki;
      wave_argmax(bv, bi);
      th = bv;
      thi = bi;
      if (bi == lane) {   // the winning lane leaves the race
        kv = -INFINITY;
        ki = kSentinelId;
      }
    }
    if (lane == 0) s_theta[w] = (thi == kSentinelId) ? -INFINITY : th;
  }
  __syncthreads();
  float theta = s_theta[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) theta = fmaxf(theta, s_theta[i]);

  if (c > 0.f && tid == 0) {
    M = sm[0];
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sm[i]);
    for (int i = 0; i < kWaves; ++i)
      if (sm[i] > -INFINITY) S += ss[i] * fast_exp2(sm[i] * c - M * c);
  }

  // ---- candidate lanes and their rank in (wave, lane) order
  const bool cand = has && tm >= theta;
  const unsigned long long bal = __ballot(cand);
  if (lane == 0) s_cnt[w] = __popcll(bal);
  if (tid < SPEC_MAX_F) {
    l_v[tid] = -INFINITY;
    l_i[tid] = kSentinelId;
  }
  __syncthreads();
  int rank = __popcll(bal & ((1ull << lane) - 1ull));
  int ncand = 0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) rank += s_cnt[i];
    ncand += s_cnt[i];
  }

  for (int b0 = 0; b0 < ncand; b0 += kCandSlots) {
    if (cand && rank >= b0 && rank < b0 + kCandSlots) {
      const int sl = rank - b0;
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i) c_vec[sl][i] = q[i];
      c_ext[sl][0] = ext[0];
      c_ext[sl][1] = ext[1];
      c_tid[sl] = tid;
    }
    __syncthreads();
    if (w == 0) {
      const int nslot = min(kCandSlots, ncand - b0);
      // decode this lane's share of the candidate elements once
      float ev[kSel + 1];
      int ei[kSel + 1];
#pragma unroll
      for (int s = 0; s < kSel; ++s) {
        const int e = lane + s * kWave;
        const int sl = e / kPer, wi = e % kPer;
        float val = -INFINITY;
        int id = kSentinelId;
        if (sl < nslot) {
          const int ct = c_tid[sl];
          if (wi < kVecPerThread * N) {
            const int i = wi / N, j = wi % N;
            const int vi = cr.vbeg + i * kBlock + ct;
            if (vi < cr.vend) {
              val = E::from_words(reinterpret_cast<const uint32_t*>(&c_vec[sl][i]), j);
              id = sp.head + vi * N + j;
            }
          } else if (wi == kVecPerThread * N) {
            if (cr.first && ct < sp.head) {
              val = c_ext[sl][0];
              id = ct;
            }
          } else if (cr.last && ct < V - sp.tail) {
            val = c_ext[sl][1];
            id = sp.tail + ct;
          }
        }
        ev[s] = val;
        ei[s] = id;
      }
      // the running list from earlier batches competes too
      ev[kSel] = lane < F ? l_v[lane] : -INFINITY;
      ei[kSel] = lane < F ? l_i[lane] : kSentinelId;
      float pv = INFINITY;
      int pi = -1;
      for (int f = 0; f < F; ++f) {
        float bv = -INFINITY;
        int bi = kSentinelId;
#pragma unroll
        for (int s = 0; s <= kSel; ++s)
          if (after(ev[s], ei[s], pv, pi) && better(ev[s], ei[s], bv, bi)) {
            bv = ev[s];
            bi = ei[s];
          }
        wave_argmax(bv, bi);
        pv = bv;
        pi = bi;
        if (lane == 0) {
          l_v[f] = bv;
          l_i[f] = bi;
        }
      }
    }
    __syncthreads();
  }

  // ---- publish the chunk's list and statistics
  const size_t pc = static_cast<size_t>(rk) * nchunk + ch;
  if (tid < F) store_coherent(&part[pc * F + tid], pack2(l_v[tid], l_i[tid]));
  if (tid == 0 && c > 0.f) store_coherent(&pstat[pc], pack2(M, S));
  if (!arrive_last(cnt, static_cast<unsigned>(nchunk), &s_flag)) return;

  // ---- last workgroup of the slot: merge the chunks' lists
  if (w != 0) return;
  const ArgPart* pr = part + static_cast<size_t>(rk) * nchunk * F;
  const int total = nchunk * F;
  float pv = INFINITY;
  int pi = -1;
  float Mr = -INFINITY;
  double Sr = 0.0;
  if (c > 0.f) {
    const float2* ps = pstat + static_cast<size_t>(rk) * nchunk;
    float lm = -INFINITY;
    for (int j = lane; j < nchunk; j += kWave) lm = fmaxf(lm, lo_float(load_coherent(&ps[j])));
    Mr = wave_max(lm);
    const float mc = Mr * c;
    double ls = 0.0;
    for (int j = lane; j < nchunk; j += kWave) {
      const uint64_t st = load_coherent(&ps[j]);
      if (lo_float(st) > -INFINITY) {
        const float qc = lo_float(st) * c;
        ls += static_cast<double>(hi_float(st)) *
              exp2(static_cast<double>(qc) - static_cast<double>(mc));
      }
    }
    Sr = wave_sum(ls);
  }
  for (int f = 0; f < F; ++f) {
    float bv = -INFINITY;
    int bi = kSentinelId;
    for (int j = lane; j < total; j += kWave) {
      const uint64_t a = load_coherent(&pr[j]);
      const float av = lo_float(a);
      const int ai = hi_int(a);
      if (after(av, ai, pv, pi) && better(av, ai, bv, bi)) {
        bv = av;
        bi = ai;
      }
    }
    wave_argmax(bv, bi);
    pv = bv;
    pi = bi;
    if (lane == 0) {
      const size_t o = static_cast<size_t>(rk) * F + f;
      out_keys[o] = bi;
      if (out_prob) {
        float pr_f;
        if (c > 0.f) {
          const float mc = Mr * c;
          pr_f = static_cast<float>(
              exp(kLn2 * (static_cast<double>(bv) * c - static_cast<double>(mc))) / Sr);
        } else {
          pr_f = f == 0 ? 1.f : 0.f;
        }
        out_prob[o] = pr_f;
      }
    }
  }
  if (lane == 0) reset_counter(cnt);
}

template <typename TIn>
int launch_predict(const void* draft, int B, int K, int V, int F, float T, int32_t* out_keys,
                   float* out_prob, void* ws, hipStream_t stream, const KernelPlan& P) {
  if (P.cv > kPassVecs) return SPEC_ERR_ARG;   // a chunk must fit one register-resident pass
  const size_t g = static_cast<size_t>(B) * K * P.nchunk;
  if (!grid_fits(g)) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, F);
  const float c = T > 0.f ? exp2_scale(T) : 0.f;
  hipLaunchKernelGGL(predict_kernel<TIn>, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0, stream,
                     static_cast<const TIn*>(draft), K, V, F, c, P.nchunk, P.cv,
                     ws_ptr<ArgPart>(ws, L.part_topf), ws_ptr<float2>(ws, L.part_pstat),
                     ws_ptr<unsigned>(ws, L.cnt_a), out_keys, out_prob);
  return launch_status();
}

}  // namespace
}  // namespace sv

extern "C" int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int K, int V,
                                     int F, float temperature, int32_t* out_keys,
                                     float* out_key_prob, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  using namespace sv;
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (F < 1 || F > SPEC_MAX_F || F > V) return SPEC_ERR_ARG;
  if (check_logits(draft_logits, dtype) != SPEC_OK || out_keys == nullptr) return SPEC_ERR_ARG;
  if (!std::isfinite(temperature) || temperature < 0.f ||
      (temperature > 0.f && !std::isfinite(exp2_scale(temperature))))
    return SPEC_ERR_TEMPERATURE;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, F)) != SPEC_OK) return rc;
  if (dtype == SPEC_BF16)
    return launch_predict<uint16_t>(draft_logits, B, K, V, F, temperature, out_keys,
                                    out_key_prob, workspace, stream, predict_plan(B, K, V, 8));
  return launch_predict<float>(draft_logits, B, K, V, F, temperature, out_keys, out_key_prob,
                               workspace, stream, predict_plan(B, K, V, 4));
}
