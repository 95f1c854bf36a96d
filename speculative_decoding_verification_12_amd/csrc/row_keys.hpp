// Row statistics and top-key selection shared by the verification and outcome-key kernels.
//
// The statistics of a logit row at temperature T (c = log2(e)/T): its maximum M and
// S = sum 2^((l - M) c), streamed in chunks (one workgroup each) and merged afterwards. The
// key selection picks a row's top tokens from the per-wave maxima that pass left behind,
// re-reading only the waves that can hold one.
#pragma once

#include "spec_common.hpp"
#include "spec_verify.h"

namespace sv {

// ------------------------------------------------------------------------------ statistics
// Folds n values into a running (m, s) where s = sum 2^((l - m) c).
// With kSum false only the maximum is kept (s stays 0).
template <bool kSum = true, int n>
__device__ __forceinline__ void absorb(const float (&v)[n], float c, float& m, float& s) {
  float bm = v[0];
#pragma unroll
  for (int j = 1; j < n; ++j) bm = fmaxf(bm, v[j]);
  if constexpr (!kSum) {
    m = fmaxf(m, bm);
    return;
  }
  if (bm > m) {
    s *= rel_exp2(m, bm, c);   // s is 0 while m is -inf, so the factor (0) is then moot
    m = bm;
  }
  // While |m c| <= 64 in every lane of the wave, each term is 2^fl(l c - fl(m c)) by one fma: the
  // reference's rounding error (|m c| 2^-24 <= 2^-18) then moves every term by less than 3e-6
  // relative. Beyond that (tiny temperatures) the gap is taken first, as rel_exp2 does.
  const float mc = m * c;
  if (__all(!(m > -INFINITY) || fabsf(mc) <= 64.f)) {
    if (m > -INFINITY) {
#pragma unroll
      for (int j = 0; j < n; ++j) s += fast_exp2(fmaf(v[j], c, -mc));
    }
  } else if (m > -INFINITY) {
#pragma unroll
    for (int j = 0; j < n; ++j) s += rel_exp2(v[j], m, c);
  }
}

// One thread's share of chunk `cr`: scalar head/tail elements, then passes of
// kVecPerThread vectors, all loads of a pass issued before any arithmetic.
// kNT reads the vectors with non-temporal loads. Whether that pays depends on what reads the rows
// again afterwards (the draw's re-read of row m, the key selection's re-read of a few waves); it
// is chosen per pass from measurements.
template <typename TIn, bool kSum = true, bool kNT = false>
__device__ __forceinline__ void thread_chunk_stats(const TIn* row, const RowSpan& sp,
                                                   const ChunkRange& cr, int V, float c,
                                                   float& m, float& s) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  const int tid = threadIdx.x;
  m = -INFINITY;
  s = 0.f;
  {
    float e[2] = {-INFINITY, -INFINITY};
    if (cr.first && tid < sp.head) e[0] = E::one(row, tid);
    if (cr.last && tid < V - sp.tail) e[1] = E::one(row, sp.tail + tid);
    absorb<kSum>(e, c, m, s);
  }
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
  for (int base = cr.vbeg; base < cr.vend; base += kPassVecs) {
    uint4 q[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int vi = base + i * kBlock + tid;
      if constexpr (kNT)
        q[i] = vi < cr.vend ? load_stream(vrow, vi) : neg_inf_vec<TIn>();
      else
        q[i] = vi < cr.vend ? vrow[vi] : neg_inf_vec<TIn>();
    }
    float v[kVecPerThread * N];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      float t[N];
      E::unpack(q[i], t);
#pragma unroll
      for (int j = 0; j < N; ++j) v[i * N + j] = t[j];
    }
    absorb<kSum>(v, c, m, s);
  }
}

// Block reduction of the threads' (m, s); the result is valid in thread 0. With `wave_max_out`,
// lane 0 of every wave also stores its wave's maximum there (indexed by wave).
__device__ __forceinline__ void block_stats(float m, float s, float c, float* sm, float* ss,
                                            float& M, float& S, float* wave_max_out = nullptr) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const float wm = wave_max(m);
  if (wave_max_out != nullptr && lane == 0) wave_max_out[w] = wm;
  const float sc = (m > -INFINITY) ? s * rel_exp2(m, wm, c) : 0.f;
  const float ws = wave_sum(sc);
  if (lane == 0) {
    sm[w] = wm;
    ss[w] = ws;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    M = sm[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) M = fmaxf(M, sm[i]);
    S = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
      if (sm[i] > -INFINITY) S += ss[i] * rel_exp2(sm[i], M, c);
  }
}

// ------------------------------------------------------------------------------ key selection
// Outcome keys from a statistics pass over the draft rows ([SSD] section "1. Outcome
// Prediction": the placed token is predicted from the draft's top logits). The pass keeps, for
// every wave of a row, the wave's maximum. Let t be the F'-th largest of these maxima (F' keys
// looked for, ties counted): F' waves hold an element >= t, so the row's F'-th largest element
// is >= t and every one of the row's top F' sits in a wave whose maximum reaches t. Only those
// waves (usually F') are read again: each wave of the selecting workgroup takes a share of them,
// lists their elements >= t in LDS (numbered by ballot), and wave 0 ranks all listed elements in
// the order (value desc, id asc); ranks 0..F'-1 are the picks.
constexpr int kSentinelId = 0x7fffffff;

__device__ __forceinline__ bool after_in_order(float v, int i, float pv, int pi) {
  return v < pv || (v == pv && i > pi);
}

__device__ __forceinline__ int lanes_below(unsigned long long bal) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(bal >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
}

// Replaces the running best (lanes 0..Fp-1 hold picks in order) by the best Fp of itself and
// the candidates each lane offers through `offer(pv, pi, bv, bi)` (its best entry after (pv, pi)).
template <typename Offer>
__device__ __forceinline__ void merge_running(float& rv, int& ri, int Fp, Offer offer) {
  const int lane = threadIdx.x & (kWave - 1);
  const float hv = lane < Fp ? rv : -INFINITY;
  const int hi = lane < Fp ? ri : kSentinelId;
  float pv = INFINITY, nv = -INFINITY;
  int pi = -1, ni = kSentinelId;
  for (int f = 0; f < Fp; ++f) {
    float bv = -INFINITY;
    int bi = kSentinelId;
    if (hi != kSentinelId && after_in_order(hv, hi, pv, pi) && better(hv, hi, bv, bi)) {
      bv = hv;
      bi = hi;
    }
    offer(pv, pi, bv, bi);
    wave_argmax(bv, bi);
    pv = bv;
    pi = bi;
    if (lane == f) {
      nv = bv;
      ni = bi;
    }
  }
  rv = nv;
  ri = ni;
}

struct RowStat {   // a row's merged statistics: max and sum of 2^((l - max) c)
  float M;
  float pad;
  double S;
};


// The keys of one row: the best Fp tokens in the order (value desc, id asc), the token xk
// skipped (xk < 0: none), the first nkeys of the rest written to keys_out[0..nkeys) with, when
// prob_out is given, q(key) = 2^((l - M) c) / S from the row's statistics (c > 0), or at
// c = 0 the temperature-zero probability: 1 for the rank-0 token, 0 for any other. The row's
// statistics come from row_stat(), called by the 64 lanes of wave 0 just before the keys are
// written (so a caller can merge them there, after its loads have long arrived).
// The row's statistics pass used chunks of cv_s vectors, nchunk_s of them, and left the maxima
// of its four waves per chunk in wmx[0 .. 4*nchunk_s). Called by all NW waves of a workgroup
// (NW * 64 threads) with uniform arguments; kCoherent reads wmx with device-coherent loads (for
// maxima written earlier by the same launch).
template <typename TIn, int NW, bool kCoherent, typename RowStatFn>
__device__ __forceinline__ void select_keys(const TIn* __restrict__ row, int V, int nchunk_s,
                                            int cv_s, const float* __restrict__ wmx, int Fp,
                                            int nkeys, int xk, RowStatFn row_stat, float c,
                                            int32_t* __restrict__ keys_out,
                                            float* __restrict__ prob_out) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  __shared__ float s_cv[NW][kWave];
  __shared__ int s_ci[NW][kWave];
  __shared__ int s_cnt[NW];
  __shared__ float s_pv[SPEC_MAX_F];
  __shared__ int s_pi[SPEC_MAX_F];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int nl = nchunk_s * kWaves;
  auto ldmax = [&](int j) { return kCoherent ? load_coherent_f32(wmx + j) : wmx[j]; };
  constexpr int kHeldMax = 4;   // wave maxima a lane keeps (lists of up to 256 waves)
  float hm[kHeldMax];
#pragma unroll
  for (int h = 0; h < kHeldMax; ++h) {
    const int j = lane + h * kWave;
    const float v = ldmax(j < nl ? j : nl - 1);   // unconditional: all loads in flight at once
    hm[h] = j < nl ? v : -INFINITY;
  }
  const bool more = nl > kHeldMax * kWave;   // uniform; longer lists are re-read

  // ---- t, the Fp-th largest wave maximum (ties counted; -inf with fewer than Fp), computed by
  // every wave alike
  float t = -INFINITY;
  {
    float pv = INFINITY;
    int pi = -1;
    for (int f = 0; f < Fp; ++f) {
      float bv = -INFINITY;
      int bi = kSentinelId;
#pragma unroll
      for (int h = 0; h < kHeldMax; ++h) {
        const int j = lane + h * kWave;
        if (j < nl && after_in_order(hm[h], j, pv, pi) && better(hm[h], j, bv, bi)) {
          bv = hm[h];
          bi = j;
        }
      }
      if (more)
        for (int j = lane + kHeldMax * kWave; j < nl; j += kWave) {
          const float v = ldmax(j);
          if (after_in_order(v, j, pv, pi) && better(v, j, bv, bi)) {
            bv = v;
            bi = j;
          }
        }
      wave_argmax(bv, bi);
      pv = bv;
      pi = bi;
      t = bi == kSentinelId ? -INFINITY : bv;
    }
  }

  // ---- every wave: its share of the chosen waves (in order, dealt out round robin). Every
  // element >= t (the row's top Fp among them) goes to the wave's LDS list, numbered by ballot
  // one column of elements at a time (a column without any costs one scalar branch). A wave
  // whose list would pass 64 entries (many elements equal to t) redoes its share exactly.
  const RowSpan sp = row_span(row, V);
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
  float rv = -INFINITY;
  int ri = kSentinelId;
  auto share = [&](auto&& chunk_fn) {
    int nchosen = 0;   // uniform
    for (int base = 0; base < nl; base += kWave) {
      const int j = base + lane;
      float mj = -INFINITY;
#pragma unroll
      for (int h = 0; h < kHeldMax; ++h)
        if (base == h * kWave) mj = hm[h];
      if (base >= kHeldMax * kWave && j < nl) mj = ldmax(j);
      const unsigned long long pick = __ballot(j < nl && mj >= t);
      for (unsigned long long m = pick; m != 0ull; m &= m - 1ull) {   // uniform
        const int jj = base + __ffsll(static_cast<long long>(m)) - 1;
        if ((nchosen++ % NW) == w) chunk_fn(jj / kWaves, jj % kWaves);
      }
    }
  };
  // the elements a statistics thread held: (ok, value, id) for each, head and tail first
  auto elements = [&](int ch, int sw, auto&& fn) {
    const ChunkRange cr = chunk_range(sp, ch, nchunk_s, cv_s);
    const int st = sw * kWave + lane;   // the statistics thread whose elements this lane takes
    const bool hh = cr.first && st < sp.head, ht = cr.last && st < V - sp.tail;
    uint32_t rh = 0u, rt = 0u;
    if ((cr.first && sp.head > 0) || (cr.last && V > sp.tail)) {   // uniform
      rh = E::raw(row, min(st, V - 1));
      rt = E::raw(row, min(sp.tail + st, V - 1));
    }
    fn(hh, hh ? E::cvt(rh) : -INFINITY, st);
    fn(ht, ht ? E::cvt(rt) : -INFINITY, sp.tail + st);
    for (int pbase = cr.vbeg; pbase < cr.vend; pbase += kPassVecs) {
      uint4 qv[kVecPerThread];
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i)
        qv[i] = vrow[min(pbase + i * kBlock + st, cr.vend - 1)];
#pragma unroll
      for (int i = 0; i < kVecPerThread; ++i) {
        const int vi = pbase + i * kBlock + st;
        float x[N];
        E::unpack(qv[i], x);
#pragma unroll
        for (int e = 0; e < N; ++e) fn(vi < cr.vend, x[e], sp.head + vi * N + e);
      }
    }
  };
  int cnt = 0;   // uniform
  share([&](int ch, int sw) {
    elements(ch, sw, [&](bool ok, float v, int id) {
      const unsigned long long bal = __ballot(ok && v >= t);
      if (bal == 0ull) return;
      const int at = cnt + lanes_below(bal);
      if (ok && v >= t && at < kWave) {
        s_cv[w][at] = v;
        s_ci[w][at] = id;
      }
      cnt += __popcll(bal);
    });
  });
  if (cnt > kWave) {   // rare: the wave's exact best Fp replace its list
    share([&](int ch, int sw) {
      merge_running(rv, ri, Fp, [&](float pv, int pi, float& bv, int& bi) {
        elements(ch, sw, [&](bool ok, float v, int id) {
          if (ok && v >= t && after_in_order(v, id, pv, pi) && better(v, id, bv, bi)) {
            bv = v;
            bi = id;
          }
        });
      });
    });
    __builtin_amdgcn_wave_barrier();
    if (lane < Fp) {
      s_cv[w][lane] = rv;
      s_ci[w][lane] = ri;
    }
    cnt = Fp;
  }
  if (lane == 0) s_cnt[w] = cnt;
  __syncthreads();
  if (w != 0) return;

  // ---- wave 0: every candidate's rank in the order (value desc, id asc) among all of them;
  // ranks 0..Fp-1 are the picks, in order. Candidate g of the lists laid end to end is entry lj
  // of list lw.
  int pre[NW + 1];   // uniform prefix sums of the list lengths
  pre[0] = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) pre[i + 1] = pre[i] + s_cnt[i];
  const int tot = pre[NW];
  for (int g0 = 0; g0 < tot; g0 += kWave) {   // uniform
    const int g = g0 + lane;
    int lw = 0, lj = g;
#pragma unroll
    for (int i = 1; i < NW; ++i)
      if (g >= pre[i]) {
        lw = i;
        lj = g - pre[i];
      }
    const bool mine = g < tot;
    const float v = mine ? s_cv[lw][lj] : -INFINITY;
    const int id = mine ? s_ci[lw][lj] : kSentinelId;
    int rank = 0;
    if (tot <= kWave) {
      // the usual case: every candidate sits in one lane, and candidate h reaches the others by
      // a lane read (no LDS round trip per compare)
      for (int h = 0; h < tot; ++h)   // uniform
        rank += better(readlane_f32(v, h), __builtin_amdgcn_readlane(id, h), v, id) ? 1 : 0;
    } else {
#pragma unroll
      for (int wl = 0; wl < NW; ++wl)
        for (int h = 0; h < pre[wl + 1] - pre[wl]; ++h)   // uniform
          rank += better(s_cv[wl][h], s_ci[wl][h], v, id) ? 1 : 0;
    }
    if (mine && rank < Fp) {
      s_pv[rank] = v;
      s_pi[rank] = id;
    }
  }
  __builtin_amdgcn_wave_barrier();
  // lane f writes pick f (one lane per key); a pick equal to xk is skipped and the later picks
  // move up by one
  const bool valid = lane < Fp && lane < tot;
  const int pid = valid ? s_pi[lane] : kSentinelId;
  const float pvv = valid ? s_pv[lane] : -INFINITY;
  const unsigned long long xm = __ballot(valid && pid == xk);
  const int xpos = xm ? __ffsll(static_cast<long long>(xm)) - 1 : kWave;
  const int pos = lane - (xpos < lane ? 1 : 0);
  const RowStat rs = row_stat();
  if (valid && lane != xpos && pos < nkeys) {
    keys_out[pos] = pid;
    if (prob_out)
      prob_out[pos] =
          c > 0.f ? static_cast<float>(
                        exp2_wide(static_cast<double>(pvv - rs.M) * static_cast<double>(c)) /
                        rs.S)
                  : (lane == 0 ? 1.f : 0.f);
  }
}

}  // namespace sv
