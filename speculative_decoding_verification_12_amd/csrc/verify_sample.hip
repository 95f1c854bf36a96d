// Speculative-sampling verification (temperature T > 0) on gfx950.
//
// Method (page "speculative decodingとは", section on how the four-stage loop works, stages 3
// and 4; page "LLMの生成を5倍速くする「D3D」を図で読む", sections 検証のしくみ① and 検証のまとめ):
// p_k = softmax(l^t_k / T) for the K+1 target rows, q_k = softmax(l^d_k / T) for the K draft
// rows; slots are scanned left to right, slot k kept iff u_k < min(1, p_k(x_k) / q_k(x_k)); at
// the first rejection m a token is drawn from max(0, p_m - q_m), or from the extra row p_K when
// every draft was kept; tau = m + 1 and the KV length advances by tau.
//
// Two launches, both HBM-streaming, no matrix cores (nothing here is a contraction):
//  1. sample_stats_kernel: one workgroup per (request, row, chunk of 16-byte vectors). Each
//     thread keeps a running max m and a sum of 2^(l*c - fl(m*c)), c = log2(e)/T, with one
//     hardware exp2 per element; wave butterflies and LDS reduce to the chunk's (M, S), written
//     with a plain store. The workgroup whose chunk holds a slot's draft token also records
//     that token's logit. No workgroup waits on another: the kernel boundary is the only
//     synchronisation.
//  2. sample_draw_kernel: one workgroup per (request, chunk of 1024 vectors). Each first merges
//     its request's chunk statistics (a few hundred bytes, identical in every workgroup of the
//     request), evaluates every slot's log-ratio in float64 and finds the first rejection m
//     with a wave ballot; chunk 0 writes tau, kv, the kept tokens and p_k(x_k), q_k(x_k). Then
//     it re-reads its chunk of row m of the target (and of the draft when m < K) and sums the
//     draw weights in float64. The request's last workgroup to arrive (device-scope counter)
//     finds the chunk that holds u*Z with one wave-wide prefix scan, rescans that chunk with a
//     block prefix sum and writes the drawn token.
#include <hip/hip_ext.h>

#include "api_common.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

// ------------------------------------------------------------------------------ statistics
// Folds n values into a running (m, s) where s = sum 2^(l*c - fl32(m*c)).
template <int n>
__device__ __forceinline__ void absorb(const float (&v)[n], float c, float& m, float& s) {
  float bm = v[0];
#pragma unroll
  for (int j = 1; j < n; ++j) bm = fmaxf(bm, v[j]);
  if (bm > m) {
    s *= fast_exp2(m * c - bm * c);   // s is 0 while m is -inf, so the factor is then moot
    m = bm;
  }
  if (m > -INFINITY) {
    const float mc = m * c;
#pragma unroll
    for (int j = 0; j < n; ++j) s += fast_exp2(fmaf(v[j], c, -mc));
  }
}

// One thread's share of chunk `cr`: scalar head/tail elements, then passes of
// kVecPerThread vectors, all loads of a pass issued before any arithmetic.
template <typename TIn>
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
    absorb(e, c, m, s);
  }
  const uint4* vrow = reinterpret_cast<const uint4*>(row + sp.head);
  for (int base = cr.vbeg; base < cr.vend; base += kPassVecs) {
    uint4 q[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
      const int vi = base + i * kBlock + tid;
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
    absorb(v, c, m, s);
  }
}

// Block reduction of the threads' (m, s); the result is valid in thread 0.
__device__ __forceinline__ void block_stats(float m, float s, float c, float* sm, float* ss,
                                            float& M, float& S) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const float wm = wave_max(m);
  const float sc = (m > -INFINITY) ? s * fast_exp2(m * c - wm * c) : 0.f;
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
      if (sm[i] > -INFINITY) S += ss[i] * fast_exp2(sm[i] * c - M * c);
  }
}

template <typename TIn>
__device__ __forceinline__ const TIn* slot_row(const TIn* tgt, const TIn* drf, int b, int r,
                                               int K, int V) {
  // rows 0..K are the request's target rows, rows K+1..2K its draft rows
  return r <= K ? tgt + (static_cast<size_t>(b) * (K + 1) + r) * static_cast<size_t>(V)
                : drf + (static_cast<size_t>(b) * K + (r - K - 1)) * static_cast<size_t>(V);
}

template <typename TIn>
__global__ __launch_bounds__(kBlock) void sample_stats_kernel(
    const TIn* __restrict__ tgt, const TIn* __restrict__ drf, const int32_t* __restrict__ xtok,
    int K, int V, float c, int nchunk, int cv, float2* __restrict__ part,
    float* __restrict__ gath) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  __shared__ float sm[kWaves], ss[kWaves];

  const int rows = 2 * K + 1;
  const int ch = blockIdx.x % nchunk;
  const int rb = blockIdx.x / nchunk;   // request-major (request, row) index
  const int r = rb % rows;
  const int b = rb / rows;

  const TIn* row = slot_row(tgt, drf, b, r, K, V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);

  // The workgroup whose chunk holds the slot's draft token also reads that token's logit, so
  // the merge finds it without another dependent load. Rows 0..K-1 are target slots, K+1..2K
  // draft slots; row K (the extra target row) has no draft token.
  const int slot = r < K ? r : r - K - 1;
  if (r != K && threadIdx.x == 0) {
    const int x = xtok[static_cast<size_t>(b) * K + slot];
    const int lo = cr.first ? 0 : sp.head + cr.vbeg * N;
    const int hi = cr.last ? V : sp.head + cr.vend * N;
    if (x >= lo && x < hi) gath[static_cast<size_t>(b) * 2 * K + (r < K ? slot : K + slot)] = E::one(row, x);
  }

  float m, s, M, S;
  thread_chunk_stats(row, sp, cr, V, c, m, s);
  block_stats(m, s, c, sm, ss, M, S);
  if (threadIdx.x == 0) part[static_cast<size_t>(rb) * nchunk + ch] = make_float2(M, S);
}

// ------------------------------------------------------------------------------ draw
// Weights of the draw over row m: w = max(0, p - q) (residual, m < K) or w = p (bonus, m == K),
// with p = 2^(l*c - mc_t) / S_t and q likewise. `use_p` switches to w = p, the fallback when
// round-off leaves no residual mass.
template <typename TIn>
struct DrawRows {
  const TIn* t;
  const TIn* d;      // draft row m (unused for the bonus row)
  RowSpan sp;        // span of the target row; chunks follow it
  bool d_aligned;    // draft row has the same 16-byte phase, so vector loads line up
  bool resid;
};

template <typename TIn>
__device__ __forceinline__ float weight_one(const DrawRows<TIn>& R, const ReqState& st, float c,
                                            int tok, bool use_p, float& p) {
  p = fast_exp2(fmaf(Elem<TIn>::one(R.t, tok), c, -st.mc_t)) * st.inv_t;
  if (!R.resid || use_p) return p;
  const float q = fast_exp2(fmaf(Elem<TIn>::one(R.d, tok), c, -st.mc_d)) * st.inv_d;
  return fmaxf(p - q, 0.f);
}

template <typename TIn>
__device__ __forceinline__ void weight_group(const DrawRows<TIn>& R, const ReqState& st, float c,
                                             const uint4& qt, const uint4& qd, int v, bool use_p,
                                             float (&w)[Elem<TIn>::N],
                                             float (&p)[Elem<TIn>::N]) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  float lt[N];
  E::unpack(qt, lt);
#pragma unroll
  for (int j = 0; j < N; ++j) p[j] = fast_exp2(fmaf(lt[j], c, -st.mc_t)) * st.inv_t;
  if (!R.resid || use_p) {
#pragma unroll
    for (int j = 0; j < N; ++j) w[j] = p[j];
    return;
  }
  float ld[N];
  if (R.d_aligned) {
    E::unpack(qd, ld);
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) ld[j] = E::one(R.d, R.sp.head + v * N + j);
  }
#pragma unroll
  for (int j = 0; j < N; ++j)
    w[j] = fmaxf(p[j] - fast_exp2(fmaf(ld[j], c, -st.mc_d)) * st.inv_d, 0.f);
}

template <typename TIn>
__device__ __forceinline__ void load_pair(const DrawRows<TIn>& R, int v, bool has, uint4& qt,
                                          uint4& qd) {
  const uint4* tv = reinterpret_cast<const uint4*>(R.t + R.sp.head);
  const uint4* dv = reinterpret_cast<const uint4*>(R.d + R.sp.head);
  qt = has ? tv[v] : neg_inf_vec<TIn>();
  qd = (has && R.resid && R.d_aligned) ? dv[v] : neg_inf_vec<TIn>();
}

// Block-wide inclusive and exclusive prefix sums in thread order. excl of thread t equals incl of
// thread t-1 bit for bit. `tot` receives the block total.
__device__ __forceinline__ void block_scan(double x, double* s_wave, double& incl, double& excl,
                                           double& tot) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const double wi = wave_inclusive_scan(x, lane);
  double we = __shfl_up(wi, 1, kWave);
  if (lane == 0) we = 0.0;
  if (lane == kWave - 1) s_wave[w] = wi;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += s_wave[i];
  double all = 0.0;
  for (int i = 0; i < kWaves; ++i) all += s_wave[i];
  incl = off + wi;
  excl = lane == 0 ? off : off + we;
  tot = all;
  __syncthreads();
}

// Chunks of at most kBlock * kDrawVecs vectors (see draw_plan).
template <typename TIn>
__global__ __launch_bounds__(kBlock) void sample_draw_kernel(
    const TIn* __restrict__ tgt, const TIn* __restrict__ drf, const int32_t* __restrict__ xtok,
    const float* __restrict__ uni, const int32_t* __restrict__ kv_in, int K, int V, float c,
    int nchunk_s, const float2* __restrict__ part_s, const float* __restrict__ gath,
    int nchunk, int cv, double2* __restrict__ part, unsigned* __restrict__ cnt_base,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_tau, int32_t* __restrict__ out_kv,
    float* __restrict__ out_p, float* __restrict__ out_q) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  __shared__ double s_a[kWaves], s_b[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ int s_flag, s_cs, s_usep, s_y, s_first;
  __shared__ double s_cum, s_t;
  __shared__ float row_m[2 * SPEC_MAX_K + 1];
  __shared__ double row_s[2 * SPEC_MAX_K + 1];
  __shared__ ReqState s_st;

  const int b = blockIdx.x / nchunk;
  const int ch = blockIdx.x % nchunk;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int rows = 2 * K + 1;

  // ---- merge the statistics pass of request b (every workgroup of b does the same, bit for
  // bit): row (max, sum) in fp32/fp64, slot log-ratios in fp64, first rejection by ballot
  {
    const bool valid = w == 0 && lane < K;
    int xk = 0;
    float lt = 0.f, ld = 0.f, uk = 0.f;
    if (valid) {
      xk = xtok[static_cast<size_t>(b) * K + lane];
      uk = uni[static_cast<size_t>(b) * (K + 1) + lane];
      lt = gath[static_cast<size_t>(b) * 2 * K + lane];
      ld = gath[static_cast<size_t>(b) * 2 * K + K + lane];
    }
    const int kv0 = (ch == 0 && tid == 0 && kv_in) ? kv_in[b] : 0;
    // Rows are merged in segments of W lanes (W = nchunk_s rounded up to a power of two, at
    // most 64), 64/W rows per wave, so one pass over the block issues every partial load at
    // once. Lanes past nchunk_s (or past the last row) carry (-inf, 0).
    int W = 1;
    while (W < nchunk_s && W < kWave) W <<= 1;
    const int per_wave = kWave / W, g = lane / W, i = lane % W;
    for (int base = 0; base < rows; base += kWaves * per_wave) {
      const int rr = base + w * per_wave + g;
      const float2* pr = part_s + (static_cast<size_t>(b) * rows + (rr < rows ? rr : 0)) * nchunk_s;
      constexpr int kHeld = 4;   // chunks a lane keeps in registers between the two passes
      float hm[kHeld], hs[kHeld];
      float lm = -INFINITY;
#pragma unroll
      for (int h = 0; h < kHeld; ++h) {
        const int j = i + h * W;
        const float2 q = (rr < rows && j < nchunk_s) ? pr[j] : make_float2(-INFINITY, 0.f);
        hm[h] = q.x;
        hs[h] = q.y;
        lm = fmaxf(lm, hm[h]);
      }
      if (rr < rows)
        for (int j = i + kHeld * W; j < nchunk_s; j += W) lm = fmaxf(lm, pr[j].x);
      const float Mr = seg_max(lm, W);
      const float mc = Mr * c;
      double ls = 0.0;
#pragma unroll
      for (int h = 0; h < kHeld; ++h)
        if (hm[h] > -INFINITY) ls += static_cast<double>(hs[h]) * fast_exp2(hm[h] * c - mc);
      if (rr < rows)
        for (int j = i + kHeld * W; j < nchunk_s; j += W) {
          const float2 q = pr[j];
          if (q.x > -INFINITY) ls += static_cast<double>(q.y) * fast_exp2(q.x * c - mc);
        }
      const double Sr = seg_sum(ls, W);
      if (i == 0 && rr < rows) {
        row_m[rr] = Mr;
        row_s[rr] = Sr;
      }
    }
    __syncthreads();
    if (w == 0) {
      // a draft token must be a token the draft could have sampled
      const bool bad = valid && (xk < 0 || xk >= V || ld == -INFINITY);
      bool keep = true;
      double lp = 0.0, lq = 0.0;
      if (valid && !bad) {
        const float mct = row_m[lane] * c, mcd = row_m[K + 1 + lane] * c;
        lp = kLn2 * (static_cast<double>(lt) * c - static_cast<double>(mct)) - log(row_s[lane]);
        lq = kLn2 * (static_cast<double>(ld) * c - static_cast<double>(mcd)) -
             log(row_s[K + 1 + lane]);
        // kept iff u < min(1, p/q); p >= q is kept for every u in [0,1)
        keep = (lp >= lq) || (static_cast<double>(uk) < exp(lp - lq));
      }
      const bool err = __ballot(bad) != 0ull;
      const unsigned long long rej = __ballot(valid && !keep);
      const int mm = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : K;
      if (ch == 0) {   // one workgroup of the request writes everything but the drawn token
        if (valid) {
          const size_t o = static_cast<size_t>(b) * K + lane;
          if (out_p) out_p[o] = err ? NAN : static_cast<float>(exp(lp));
          if (out_q) out_q[o] = err ? NAN : static_cast<float>(exp(lq));
        }
        for (int j = lane; j <= K; j += kWave)
          if (err || j != mm) out_tok[static_cast<size_t>(b) * (K + 1) + j] = (!err && j < mm) ? xk : -1;
        if (lane == 0) {
          out_tau[b] = err ? -1 : mm + 1;
          if (out_kv) out_kv[b] = err ? kv0 : kv0 + mm + 1;
        }
      }
      if (lane == 0) {
        ReqState st;
        st.m = err ? -1 : mm;
        st.pad = 0;
        st.mc_t = row_m[mm] * c;
        st.inv_t = static_cast<float>(1.0 / row_s[mm]);
        st.mc_d = mm < K ? row_m[K + 1 + mm] * c : 0.f;
        st.inv_d = mm < K ? static_cast<float>(1.0 / row_s[K + 1 + mm]) : 0.f;
        s_st = st;
      }
    }
    __syncthreads();
  }
  const ReqState st = s_st;
  if (st.m < 0) return;   // row error: nothing to draw (every workgroup of b agrees)
  unsigned* cnt = cnt_base + static_cast<size_t>(b) * kCounterStride;

  DrawRows<TIn> R;
  R.resid = st.m < K;
  R.t = tgt + (static_cast<size_t>(b) * (K + 1) + st.m) * static_cast<size_t>(V);
  R.d = R.resid ? drf + (static_cast<size_t>(b) * K + st.m) * static_cast<size_t>(V) : R.t;
  R.sp = row_span(R.t, V);
  R.d_aligned = row_span(R.d, V).head == R.sp.head;

  // ---- chunk masses: sum of w (draw weights) and of p (fallback weights). Thread t owns the
  // kDrawVecs adjacent vectors vbeg + t*kDrawVecs + i, plus head (first chunk) or tail (last
  // chunk) element t.
  {
    const ChunkRange cr = chunk_range(R.sp, ch, nchunk, cv);
    uint4 qt[kDrawVecs], qd[kDrawVecs];
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      const int v = cr.vbeg + tid * kDrawVecs + i;
      load_pair(R, v, v < cr.vend, qt[i], qd[i]);
    }
    double rs = 0.0, ps = 0.0;
    float p;
    if (cr.first && tid < R.sp.head) {
      rs += weight_one(R, st, c, tid, false, p);
      ps += p;
    }
    if (cr.last && tid < V - R.sp.tail) {
      rs += weight_one(R, st, c, R.sp.tail + tid, false, p);
      ps += p;
    }
    float ws = 0.f, pss = 0.f;
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      const int v = cr.vbeg + tid * kDrawVecs + i;
      if (v < cr.vend) {
        float wv[N], pv[N];
        weight_group(R, st, c, qt[i], qd[i], v, false, wv, pv);
#pragma unroll
        for (int j = 0; j < N; ++j) {
          ws += wv[j];
          pss += pv[j];
        }
      }
    }
    rs += ws;
    ps += pss;
    rs = wave_sum(rs);
    ps = wave_sum(ps);
    if (lane == 0) {
      s_a[w] = rs;
      s_b[w] = ps;
    }
    __syncthreads();
    if (tid == 0) {
      double R0 = 0.0, P0 = 0.0;
      for (int i = 0; i < kWaves; ++i) {
        R0 += s_a[i];
        P0 += s_b[i];
      }
      double2* dst = &part[static_cast<size_t>(b) * nchunk + ch];
      store_coherent(&dst->x, dbits(R0));
      store_coherent(&dst->y, dbits(P0));
    }
  }
  if (!arrive_last(cnt, static_cast<unsigned>(nchunk), &s_flag)) return;

  // ---- last workgroup of request b: find the chunk holding u*Z with one wave-wide scan
  if (w == 0) {
    const double u = static_cast<double>(uni[static_cast<size_t>(b) * (K + 1) + K]);
    const double2* pr = part + static_cast<size_t>(b) * nchunk;
    const int per = (nchunk + kWave - 1) / kWave;   // lane l owns chunks [l*per, l*per + per)
    const int j0 = min(lane * per, nchunk), j1 = min(j0 + per, nchunk);
    double rl = 0.0, pl = 0.0;
    int lastpos_r = -1, lastpos_p = -1;
    for (int j = j0; j < j1; ++j) {
      const double rj = bits_d(load_coherent(&pr[j].x));
      const double pj = bits_d(load_coherent(&pr[j].y));
      rl += rj;
      pl += pj;
      if (rj > 0.0) lastpos_r = j;
      if (pj > 0.0) lastpos_p = j;
    }
    const double ri = wave_inclusive_scan(rl, lane), pi = wave_inclusive_scan(pl, lane);
    const double rz = __shfl(ri, kWave - 1, kWave);
    const bool usep = !(rz > 0.0);   // no residual mass left by round-off: draw from p
    const double incl = usep ? pi : ri;
    const double Z = usep ? __shfl(pi, kWave - 1, kWave) : rz;
    const double t = u * Z;
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    const unsigned long long cross = __ballot(incl > t);
    int cs = -1;
    double cum = 0.0;
    if (cross) {
      const int L = __ffsll(static_cast<long long>(cross)) - 1;
      if (lane == L) {
        cum = excl;
        for (int j = j0; j < j1; ++j) {
          const double mj = bits_d(load_coherent(usep ? &pr[j].y : &pr[j].x));
          if (cum + mj > t) {
            cs = j;
            break;
          }
          cum += mj;
        }
        if (cs < 0) cs = usep ? lastpos_p : lastpos_r;   // round-off inside this lane's chunks
        if (cs < 0) cs = j1 - 1;
      }
      cs = __shfl(cs, L, kWave);
      cum = __shfl(cum, L, kWave);
    } else {   // round-off: the last chunk with positive mass (the chunk scan falls back too)
      const int lp = wave_max(usep ? lastpos_p : lastpos_r);
      cs = lp >= 0 ? lp : nchunk - 1;
    }
    if (lane == 0) {
      s_cs = cs;
      s_usep = usep ? 1 : 0;
      s_cum = cum;
      s_t = t;
      s_y = -1;
    }
  }
  __syncthreads();

  // ---- rescan the chosen chunk in token order (thread t: vectors t*kDrawVecs .. +kDrawVecs-1)
  const bool use_p = s_usep != 0;
  const double t = s_t;
  const ChunkRange cr = chunk_range(R.sp, s_cs, nchunk, cv);
  uint4 qt[kDrawVecs], qd[kDrawVecs];
#pragma unroll
  for (int i = 0; i < kDrawVecs; ++i) {
    const int v = cr.vbeg + tid * kDrawVecs + i;
    load_pair(R, v, v < cr.vend, qt[i], qd[i]);
  }
  int lastpos = -1;   // last token of positive weight this thread saw (round-off fallback)

  if (cr.first && tid == 0) {   // head elements come first
    double cum = s_cum;
    float p;
    for (int e = 0; e < R.sp.head; ++e) {
      const float we = weight_one(R, st, c, e, use_p, p);
      if (we > 0.f) lastpos = e;
      if (s_y < 0 && cum + static_cast<double>(we) > t) s_y = e;
      cum += static_cast<double>(we);
    }
    s_cum = cum;
  }
  __syncthreads();
  double cum = s_cum;
  if (s_y < 0) {   // uniform: read after a barrier
    float wv[kDrawVecs][N];
    float vs = 0.f;
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      const int v = cr.vbeg + tid * kDrawVecs + i;
      float pv[N];
      if (v < cr.vend) {
        weight_group(R, st, c, qt[i], qd[i], v, use_p, wv[i], pv);
#pragma unroll
        for (int j = 0; j < N; ++j) {
          vs += wv[i][j];
          if (wv[i][j] > 0.f) lastpos = R.sp.head + v * N + j;
        }
      } else {
#pragma unroll
        for (int j = 0; j < N; ++j) wv[i][j] = 0.f;
      }
    }
    double incl, excl, tot;
    block_scan(static_cast<double>(vs), s_a, incl, excl, tot);
    const bool crossv = cum + incl > t && vs > 0.f;
    const unsigned long long bal = __ballot(crossv);
    if (lane == 0) s_i[w] = bal ? w * kWave + __ffsll(static_cast<long long>(bal)) - 1 : -1;
    __syncthreads();
    if (tid == 0) {
      int f = -1;
      for (int i = kWaves - 1; i >= 0; --i)
        if (s_i[i] >= 0) f = s_i[i];
      s_first = f;
    }
    __syncthreads();
    if (s_first >= 0 && tid == s_first) {
      const double cb = cum + excl;
      float psum = 0.f;
      int y = -1, lp = -1;
#pragma unroll
      for (int i = 0; i < kDrawVecs; ++i) {
        const int tok0 = R.sp.head + (cr.vbeg + tid * kDrawVecs + i) * N;
#pragma unroll
        for (int j = 0; j < N; ++j) {
          psum += wv[i][j];
          if (wv[i][j] > 0.f) lp = tok0 + j;
          if (y < 0 && cb + static_cast<double>(psum) > t) y = tok0 + j;
        }
      }
      s_y = y >= 0 ? y : lp;
    }
    cum += tot;
  }
  __syncthreads();

  if (s_y < 0 && cr.last && tid == 0) {   // tail elements come last
    float p;
    for (int e = R.sp.tail; e < V; ++e) {
      const float we = weight_one(R, st, c, e, use_p, p);
      if (we > 0.f) lastpos = e;
      if (s_y < 0 && cum + static_cast<double>(we) > t) s_y = e;
      cum += static_cast<double>(we);
    }
  }
  __syncthreads();
  if (s_y < 0) {   // round-off fallback: the last token of positive weight in the chunk
    const int lp = wave_max(lastpos);
    if (lane == 0) s_i[w] = lp;
    __syncthreads();
    if (tid == 0) {
      int f = -1;
      for (int i = 0; i < kWaves; ++i) f = max(f, s_i[i]);
      s_y = f >= 0 ? f : 0;
    }
    __syncthreads();
  }
  if (tid == 0) {
    out_tok[static_cast<size_t>(b) * (K + 1) + st.m] = s_y;
    reset_counter(cnt);
  }
}

struct SamplePlan {
  KernelPlan stats, draw;
};

template <typename TIn>
SamplePlan default_sample_plan(int B, int K, int V) {
  constexpr int N = 16 / sizeof(TIn);
  return SamplePlan{stats_plan(B, K, V, N), draw_plan(B, K, V, N)};
}

template <typename TIn>
int launch_sample(const void* target, const void* draft, const int32_t* xtok, const float* uni,
                  const int32_t* kv_in, int B, int K, int V, float T, int32_t* out_tok,
                  int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                  hipStream_t stream, hipEvent_t* ev, const SamplePlan& P) {
  const size_t g1 = static_cast<size_t>(B) * (2 * K + 1) * P.stats.nchunk;
  const size_t g2 = static_cast<size_t>(B) * P.draw.nchunk;
  if (!grid_fits(g1) || !grid_fits(g2) || P.draw.cv > kBlock * kDrawVecs) return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1);
  const float c = exp2_scale(T);
  const TIn* t = static_cast<const TIn*>(target);
  const TIn* d = static_cast<const TIn*>(draft);
  float2* part1 = ws_ptr<float2>(ws, L.part_stats);
  float* gath = ws_ptr<float>(ws, L.gathered);
  double2* part2 = ws_ptr<double2>(ws, L.part_draw);
  unsigned* cnt2 = ws_ptr<unsigned>(ws, L.cnt_b);
  const dim3 grid1(static_cast<unsigned>(g1)), grid2(static_cast<unsigned>(g2)), block(kBlock);
  const int ns = P.stats.nchunk, cs = P.stats.cv, nd = P.draw.nchunk, cd = P.draw.cv;
  if (ev == nullptr) {
    hipLaunchKernelGGL(sample_stats_kernel<TIn>, grid1, block, 0, stream, t, d, xtok, K, V, c, ns,
                       cs, part1, gath);
    hipLaunchKernelGGL(sample_draw_kernel<TIn>, grid2, block, 0, stream, t, d, xtok, uni, kv_in,
                       K, V, c, ns, static_cast<const float2*>(part1),
                       static_cast<const float*>(gath), nd, cd, part2, cnt2, out_tok, out_tau,
                       out_kv, out_p, out_q);
  } else {
    // profiling: the runtime records the events at each kernel's start and end
    hipExtLaunchKernelGGL(sample_stats_kernel<TIn>, grid1, block, 0, stream, ev[0], ev[1], 0, t,
                          d, xtok, K, V, c, ns, cs, part1, gath);
    hipExtLaunchKernelGGL(sample_draw_kernel<TIn>, grid2, block, 0, stream, ev[2], ev[3], 0, t, d,
                          xtok, uni, kv_in, K, V, c, ns, static_cast<const float2*>(part1),
                          static_cast<const float*>(gath), nd, cd, part2, cnt2, out_tok, out_tau,
                          out_kv, out_p, out_q);
  }
  return launch_status();
}

int verify_sample_entry(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        const int32_t* kv_len_in, int B, int K, int V, float temperature,
                        int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                        float* out_q, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t* events) {
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (check_logits(target_logits, dtype) != SPEC_OK ||
      check_logits(draft_logits, dtype) != SPEC_OK || draft_tokens == nullptr ||
      uniforms == nullptr || out_tokens == nullptr || out_tau == nullptr)
    return SPEC_ERR_ARG;
  if (!std::isfinite(temperature) || !(temperature > 0.f) ||
      !std::isfinite(exp2_scale(temperature)))
    return SPEC_ERR_TEMPERATURE;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, 1)) != SPEC_OK) return rc;
  if (events != nullptr)
    for (int i = 0; i < 4; ++i)
      if (events[i] == nullptr) return SPEC_ERR_ARG;
  if (dtype == SPEC_BF16)
    return launch_sample<uint16_t>(target_logits, draft_logits, draft_tokens, uniforms, kv_len_in,
                                   B, K, V, temperature, out_tokens, out_tau, out_kv_len, out_p,
                                   out_q, workspace, stream, events,
                                   default_sample_plan<uint16_t>(B, K, V));
  return launch_sample<float>(target_logits, draft_logits, draft_tokens, uniforms, kv_len_in, B,
                              K, V, temperature, out_tokens, out_tau, out_kv_len, out_p, out_q,
                              workspace, stream, events, default_sample_plan<float>(B, K, V));
}

}  // namespace
}  // namespace sv

extern "C" int spec_verify_sample(const void* target_logits, const void* draft_logits,
                                  int dtype, const int32_t* draft_tokens, const float* uniforms,
                                  const int32_t* kv_len_in, int B, int K, int V,
                                  float temperature, int32_t* out_tokens, int32_t* out_tau,
                                  int32_t* out_kv_len, float* out_p, float* out_q,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sv::verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                 kv_len_in, B, K, V, temperature, out_tokens, out_tau,
                                 out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
                                 nullptr);
}

extern "C" int spec_verify_sample_timed(const void* target_logits, const void* draft_logits,
                                        int dtype, const int32_t* draft_tokens,
                                        const float* uniforms, const int32_t* kv_len_in, int B,
                                        int K, int V, float temperature, int32_t* out_tokens,
                                        int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                                        float* out_q, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return SPEC_ERR_ARG;
  return sv::verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                 kv_len_in, B, K, V, temperature, out_tokens, out_tau,
                                 out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
                                 events);
}
