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
// One launch: a workgroup of four independent waves per (request, slot, chunk of at most
// kPredictVecs 16-byte vectors). Lane t of wave w reads vectors vbeg + p*1024 + i*256 + 64w + t
// (pass p < kPredictPasses, i < 4), all issued at once, plus one head and one tail element.
// Each wave works on its own, with no LDS and no barriers:
//   1. the lane maximum, and at T > 0 the lane's online sum of 2^(l*c - fl(m*c)) against its
//      running max m (one exp per element), reduced to the wave's (max, sum);
//   2. theta: the wave's F-th largest lane maximum, ties counted. F lanes hold an element
//      >= theta, so every element of the wave's top F is >= theta, and only lanes whose maximum
//      reaches theta can hold one: usually a handful;
//   3. those lanes' elements are read again (cache hits), one element per lane of the wave; the
//      elements >= theta are numbered by ballot and published as the wave's candidate list.
//      More than kWaveSlots of them (ties at theta) and the wave publishes its exact top F
//      instead, merging the qualifying lanes' elements one lane at a time by F rounds of
//      (value, id) argmax.
// The wave counts itself in on the slot's counter; the slot's last wave selects the F best of all
// published lists by F rounds of argmax, each excluding everything at or before the previous
// pick in the order (value desc, id asc), and writes the keys and q_k(key). With the draft token
// excluded, a slot looks for F_k + 1 tokens and drops x_k (or, when x_k is not among them, the
// last one).
#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

constexpr int kSentinelId = 0x7fffffff;
constexpr int kWaveSlots = 16;  // candidates a wave publishes before falling back to its top F
constexpr int kListSlots = 16;  // entries of a wave's list: kWaveSlots, or F <= SPEC_MAX_F

// after (pv, pi) in the order (value desc, id asc)
__device__ __forceinline__ bool after(float v, int i, float pv, int pi) {
  return v < pv || (v == pv && i > pi);
}

// index of the n-th (0-based) set bit of a uniform mask, -1 if there are fewer
__device__ __forceinline__ int nth_bit(unsigned long long m, int n) {
  for (int i = 0; i < n && m != 0ull; ++i) m &= m - 1ull;
  return m != 0ull ? __ffsll(static_cast<long long>(m)) - 1 : -1;
}

// Per-slot work of one launch, passed by value: slot k < P looks for pick[k] tokens and writes
// count[k] keys at offset off[k] of its request's S keys (pick = count, or count + 1 when the
// draft token is excluded; 0 skips the slot).
struct FanoutTable {
  int P;
  int S;
  int8_t pick[SPEC_MAX_K];
  int8_t count[SPEC_MAX_K];
  int16_t off[SPEC_MAX_K];
};

template <typename TIn>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(8, 8))) void predict_kernel(
    const TIn* __restrict__ drf, const int32_t* __restrict__ xtok, int K, int V, FanoutTable ft,
    float c, int nchunk, int cv, ArgPart* __restrict__ part, int* __restrict__ pcnt,
    float2* __restrict__ pstat, unsigned* __restrict__ cnt_base, int32_t* __restrict__ out_keys,
    float* __restrict__ out_prob) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  constexpr int kVecs = kPredictPasses * kVecPerThread;   // vectors a lane reads
  constexpr int kLaneElems = kVecs * N;                    // their elements (64 or 32)
  constexpr int kGroups = kWave / kLaneElems;              // qualifying lanes per re-read (1 or 2)
  static_assert(kWave % kLaneElems == 0, "a lane's elements fit the wave");
  static_assert(SPEC_MAX_F <= kListSlots && kWaveSlots <= kListSlots, "list sizes");

  const int ch = blockIdx.x % nchunk;
  const int rk = blockIdx.x / nchunk;   // b * P + k
  const int k = rk % ft.P, b = rk / ft.P;
  const int F = ft.pick[k];   // tokens this slot looks for
  if (F == 0) return;         // the whole slot is skipped
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  unsigned* cnt = cnt_base + static_cast<size_t>(rk) * kCounterStride;
  const TIn* row = drf + (static_cast<size_t>(b) * K + k) * static_cast<size_t>(V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);   // cv <= kPredictVecs
  // vector v (0..kVecs-1) of lane tid
  auto vec_index = [&](int v, int t) { return cr.vbeg + v * kBlock + t; };

  // ---- the lane's elements, all loads in flight at once (padding is -inf)
  uint4 q[kVecs];
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
#pragma unroll
  for (int v = 0; v < kVecs; ++v) {
    const int vi = vec_index(v, tid);
    q[v] = vi < cr.vend ? vrow[vi] : neg_inf_vec<TIn>();
  }
  const bool has_head = cr.first && tid < sp.head;
  const bool has_tail = cr.last && tid < V - sp.tail;
  const float eh = has_head ? E::one(row, tid) : -INFINITY;
  const float et = has_tail ? E::one(row, sp.tail + tid) : -INFINITY;
  const bool has = has_head || has_tail || (cr.vbeg + tid < cr.vend);

  // lane maximum, and at T > 0 the online sum of 2^(l*c - fl(m*c)) against the running max m
  float tm = fmaxf(eh, et), s = 0.f;
  if (c > 0.f && tm > -INFINITY) {
    const float mc = tm * c;
    s = fast_exp2(fmaf(eh, c, -mc)) + fast_exp2(fmaf(et, c, -mc));
  }
#pragma unroll
  for (int v = 0; v < kVecs; ++v) {
    float t[N];
    E::unpack(q[v], t);
    float bm = t[0];
#pragma unroll
    for (int j = 1; j < N; ++j) bm = fmaxf(bm, t[j]);
    if (c > 0.f) {
      if (bm > tm) {
        s *= fast_exp2(tm * c - bm * c);   // s is 0 while tm is -inf
        tm = bm;
      }
      if (tm > -INFINITY) {
        const float mc = tm * c;
#pragma unroll
        for (int j = 0; j < N; ++j) s += fast_exp2(fmaf(t[j], c, -mc));
      }
    } else {
      tm = fmaxf(tm, bm);
    }
  }
  const size_t pw = (static_cast<size_t>(rk) * nchunk + ch) * kWaves + w;   // this wave's list
  if (c > 0.f) {   // the wave's (max, scaled sum) for q_k(key)
    const float wm = wave_max(tm);
    const float sc = (tm > -INFINITY) ? s * fast_exp2(tm * c - wm * c) : 0.f;
    const float wsum = wave_sum(sc);
    if (lane == 0) store_coherent(&pstat[pw], pack2(wm, wsum));
  }

  // ---- theta: the wave's F-th largest lane maximum, ties counted (-inf when fewer than F
  // lanes hold elements)
  float theta = -INFINITY;
  {
    float cur = has ? tm : -INFINITY;
    bool in = has;
    int need = F;
    while (need > 0) {   // uniform: every quantity below is wave-wide
      if (__ballot(in) == 0ull) {
        theta = -INFINITY;
        break;
      }
      const float mx = wave_max(in ? cur : -INFINITY);
      const bool at = in && cur == mx;
      need -= __popcll(__ballot(at));
      theta = mx;
      if (at) in = false;
    }
  }

  // ---- candidates: elements >= theta of the qualifying lanes, numbered by ballot. Lane j reads
  // element j % kLaneElems of the (j / kLaneElems)-th qualifying lane of a batch.
  ArgPart* list = part + pw * kListSlots;
  int count = 0;   // uniform
  auto publish = [&](bool cand, float v, int id) {
    const unsigned long long bal = __ballot(cand);
    const int slot = count + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                 static_cast<uint32_t>(bal >> 32),
                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
    if (cand && slot < kWaveSlots) store_coherent(&list[slot], pack2(v, id));
    count += __popcll(bal);
  };
  const int g = lane / kLaneElems, e = lane % kLaneElems;
  const int ev_ = e / N, el = e % N;   // the element this lane reads: vector ev_, element el
  // the qualifying lane L's element read by this lane: (in range, value, id)
  auto reread = [&](int L, bool& ok, float& v, int& id) {
    const int vi = vec_index(ev_, w * kWave + L);
    ok = L >= 0 && vi < cr.vend;
    id = sp.head + vi * N + el;
    v = ok ? E::one(row, id) : -INFINITY;
  };
  const unsigned long long qual0 = __ballot(has && tm >= theta);
  publish(has_head && eh >= theta, eh, tid);
  unsigned long long qual = qual0;
  while (qual != 0ull) {   // uniform; kGroups qualifying lanes per read
    bool ok;
    float v;
    int id;
    reread(nth_bit(qual, g), ok, v, id);
    publish(ok && v >= theta, v, id);
    for (int r = 0; r < kGroups && qual != 0ull; ++r) qual &= qual - 1ull;
  }
  publish(has_tail && et >= theta, et, sp.tail + tid);

  if (count > kWaveSlots) {
    // ---- ties at theta: the wave's exact top F, kept in lanes 0..F-1 and merged with each
    // qualifying lane's elements (and the head/tail elements) by F rounds of argmax
    float my_v = -INFINITY;
    int my_i = kSentinelId;
    auto merge_in = [&](float v, int id) {   // v, id: this lane's contender (or -inf)
      float pv = INFINITY, nv = -INFINITY;
      int pi = -1, ni = kSentinelId;
      const float hv = lane < F ? my_v : -INFINITY;
      const int hi = lane < F ? my_i : kSentinelId;
      for (int f = 0; f < F; ++f) {
        float bv = -INFINITY;
        int bi = kSentinelId;
        if (after(v, id, pv, pi) && better(v, id, bv, bi)) {
          bv = v;
          bi = id;
        }
        if (after(hv, hi, pv, pi) && better(hv, hi, bv, bi)) {
          bv = hv;
          bi = hi;
        }
        wave_argmax(bv, bi);
        pv = bv;
        pi = bi;
        if (lane == f) {
          nv = bv;
          ni = bi;
        }
      }
      my_v = nv;
      my_i = ni;
    };
    merge_in(has_head && eh >= theta ? eh : -INFINITY, has_head && eh >= theta ? tid : kSentinelId);
    merge_in(has_tail && et >= theta ? et : -INFINITY,
             has_tail && et >= theta ? sp.tail + tid : kSentinelId);
    for (unsigned long long qm = qual0; qm != 0ull;) {   // uniform
      bool ok;
      float v;
      int id;
      reread(nth_bit(qm, g), ok, v, id);
      const bool cand = ok && v >= theta;
      merge_in(cand ? v : -INFINITY, cand ? id : kSentinelId);
      for (int r = 0; r < kGroups && qm != 0ull; ++r) qm &= qm - 1ull;
    }
    if (lane < F) store_coherent(&list[lane], pack2(my_v, my_i));
    count = F;
  }
  if (lane == 0) store_coherent_u32(&pcnt[pw], static_cast<uint32_t>(count));

  // ---- count this wave in; the slot's last wave merges
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores are at the coherence point
  unsigned prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  const int nl = nchunk * kWaves;   // lists of this slot
  if (prev != static_cast<unsigned>(nl) - 1u) return;

  const size_t p0 = static_cast<size_t>(rk) * nchunk * kWaves;
  float Mr = -INFINITY;
  double Sr = 0.0;
  if (c > 0.f) {
    constexpr int kHeldStats = 4;   // wave statistics a lane keeps between the two passes
    float hm[kHeldStats], hs[kHeldStats];
    float lm = -INFINITY;
#pragma unroll
    for (int h = 0; h < kHeldStats; ++h) {
      const int j = lane + h * kWave;
      const uint64_t st = j < nl ? load_coherent(&pstat[p0 + j]) : pack2(-INFINITY, 0.f);
      hm[h] = lo_float(st);
      hs[h] = hi_float(st);
      lm = fmaxf(lm, hm[h]);
    }
    for (int j = lane + kHeldStats * kWave; j < nl; j += kWave)
      lm = fmaxf(lm, lo_float(load_coherent(&pstat[p0 + j])));
    Mr = wave_max(lm);
    const float mc = Mr * c;
    double ls = 0.0;
#pragma unroll
    for (int h = 0; h < kHeldStats; ++h)
      if (hm[h] > -INFINITY) ls += static_cast<double>(hs[h]) * fast_exp2(hm[h] * c - mc);
    for (int j = lane + kHeldStats * kWave; j < nl; j += kWave) {
      const uint64_t st = load_coherent(&pstat[p0 + j]);
      if (lo_float(st) > -INFINITY)
        ls += static_cast<double>(hi_float(st)) * fast_exp2(lo_float(st) * c - mc);
    }
    Sr = wave_sum(ls);
  }

  // The slot's lists are adjacent: nl lists of kListSlots entries. Entry g (list g / kListSlots,
  // position g % kListSlots) is valid below its list's count. Lane l holds entries l + 64h for
  // h < kHeld in registers (coalesced reads); a slot with more lists re-reads the rest every round.
  constexpr int kHeld = 8;
  const int total = nl * kListSlots;
  const ArgPart* lists = part + p0 * kListSlots;
  const int my_cnt = lane < nl ? min(static_cast<int>(load_coherent_u32(&pcnt[p0 + lane])), kListSlots)
                               : 0;   // lane l: count of list l (l < 64)
  float ev[kHeld];
  int ei[kHeld];
#pragma unroll
  for (int h = 0; h < kHeld; ++h) {
    const int gi = lane + h * kWave;
    const uint64_t a = gi < total ? load_coherent(&lists[gi]) : pack2(-INFINITY, kSentinelId);
    ev[h] = lo_float(a);
    ei[h] = hi_int(a);
  }
#pragma unroll
  for (int h = 0; h < kHeld; ++h) {   // lists 0..63 are covered by the counts in the lanes
    const int gi = lane + h * kWave;
    const int j = gi / kListSlots;
    const int cj = __shfl(my_cnt, j < kWave ? j : 0, kWave);
    if (!(gi < total && j < kWave && gi % kListSlots < cj)) {
      ev[h] = -INFINITY;
      ei[h] = kSentinelId;
    }
  }
  const bool more = total > kHeld * kWave;   // uniform
  const int xk = xtok ? xtok[static_cast<size_t>(b) * K + k] : -1;   // excluded token, if any
  const int nkeys = ft.count[k];
  const size_t obase = static_cast<size_t>(b) * ft.S + ft.off[k];
  int j = 0;   // keys written so far (uniform)
  float pv = INFINITY;
  int pi = -1;
  for (int f = 0; f < F; ++f) {
    float bv = -INFINITY;
    int bi = kSentinelId;
    auto consider = [&](float v, int id) {
      if (after(v, id, pv, pi) && better(v, id, bv, bi)) {
        bv = v;
        bi = id;
      }
    };
#pragma unroll
    for (int h = 0; h < kHeld; ++h) consider(ev[h], ei[h]);
    if (more) {   // entries beyond the registers (and lists past the 64th, with their counts)
      for (int gi = lane + kHeld * kWave; gi < total; gi += kWave) {
        const int j = gi / kListSlots;
        const int cj = min(static_cast<int>(load_coherent_u32(&pcnt[p0 + j])), kListSlots);
        if (gi % kListSlots < cj) {
          const uint64_t a = load_coherent(&lists[gi]);
          consider(lo_float(a), hi_int(a));
        }
      }
    }
    wave_argmax(bv, bi);
    pv = bv;
    pi = bi;
    if (bi == xk) continue;   // the draft token itself: never the placed token after a rejection
    if (j == nkeys) break;
    const size_t o = obase + j;
    ++j;
    if (lane == 0) {
      out_keys[o] = bi;
      if (out_prob) {
        float pr_f;
        if (c > 0.f)
          pr_f = static_cast<float>(
              exp2_wide(static_cast<double>(bv) * c - static_cast<double>(Mr * c)) / Sr);
        else
          pr_f = f == 0 ? 1.f : 0.f;
        out_prob[o] = pr_f;
      }
    }
  }
  if (lane == 0) reset_counter(cnt);
}

template <typename TIn>
int launch_predict(const void* draft, const int32_t* xtok, int B, int K, int V,
                   const FanoutTable& ft, float T, int32_t* out_keys, float* out_prob, void* ws,
                   hipStream_t stream) {
  // chunking as for all K slots of every request, so the workspace sized by
  // spec_workspace_bytes(B, K, V, .) covers any P <= K
  const KernelPlan P = predict_plan(B, K, V, 16 / static_cast<int>(sizeof(TIn)));
  if (P.cv > kPredictVecs) return SPEC_ERR_ARG;   // a chunk is one round of loads per lane
  const size_t g = static_cast<size_t>(B) * ft.P * P.nchunk;
  if (!grid_fits(g)) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1);
  const float c = T > 0.f ? exp2_scale(T) : 0.f;
  hipLaunchKernelGGL(predict_kernel<TIn>, dim3(static_cast<unsigned>(g)), dim3(kBlock), 0, stream,
                     static_cast<const TIn*>(draft), xtok, K, V, ft, c, P.nchunk, P.cv,
                     ws_ptr<ArgPart>(ws, L.part_topf), ws_ptr<int>(ws, L.part_pcnt),
                     ws_ptr<float2>(ws, L.part_pstat),
                     ws_ptr<unsigned>(ws, L.cnt_a), out_keys, out_prob);
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
                void* workspace, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return launch_predict<uint16_t>(draft_logits, xtok, B, K, V, ft, temperature, out_keys,
                                    out_key_prob, workspace, stream);
  return launch_predict<float>(draft_logits, xtok, B, K, V, ft, temperature, out_keys,
                               out_key_prob, workspace, stream);
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
    ft.pick[k] = static_cast<int8_t>(pick);
    ft.count[k] = static_cast<int8_t>(F);
    ft.off[k] = static_cast<int16_t>(ft.S);
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
                     out_key_prob, workspace, stream);
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
                     out_key_prob, workspace, stream);
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
