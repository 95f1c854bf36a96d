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
//     thread keeps a running max m and a sum of 2^((l - m) c), c = log2(e)/T, with one
//     hardware exp2 per element; wave butterflies and LDS reduce to the chunk's (M, S), written
//     with a plain store. The workgroup whose chunk holds a slot's draft token also records
//     that token's logit. No workgroup waits on another: the kernel boundary is the only
//     synchronisation. The first workgroups also clear the draw's published-mass words.
//  2. sample_draw_kernel: one workgroup per (request, chunk of 1024 vectors). Each first merges
//     its request's chunk statistics (a few hundred bytes, identical in every workgroup of the
//     request), evaluates every slot's acceptance ratio and finds the first rejection m with a
//     wave ballot; chunk 0 writes tau, kv, the kept tokens and p_k(x_k), q_k(x_k). Then it
//     re-reads its chunk of row m of the target (and of the draft when m < K), sums the draw
//     weights per thread and per chunk and publishes the chunk's mass, tagged as written. Every
//     workgroup of the request gathers all chunk masses, runs the same float64 prefix scan and
//     so learns which chunk holds u*Z; that chunk's own workgroup finds the thread (block scan
//     of the thread masses), then the token among that thread's few vectors. While one
//     workgroup per chunk fits on the GPU, the workgroup keeps its vectors in registers and
//     takes the block scan while the other masses arrive, every wave runs the chunk scan
//     itself, and the owner's search runs in the one wave holding u*Z, with no workgroup
//     barrier after the exchange; otherwise each workgroup takes several chunks and the owner
//     reads its vectors again. A workgroup that has polled for a mass too long computes that
//     chunk's mass itself (bit for bit what its owner publishes), so no workgroup ever waits on
//     one that has not been scheduled.
//     When every draft was kept and the statistics pass cut the extra row into the draw's
//     chunks, the chunk masses come from its partials instead: nothing is re-read but the
//     chunk holding u*Z, and nothing is exchanged.
// Small batches (every workgroup of both fitting on the GPU at once) run both as one launch,
// sample_fused_kernel, with the same arithmetic and the kernel boundary replaced by tagged words.
// With outcome keys (kKeys) the statistics pass also keeps the draft rows' wave maxima, and the
// draw's grid has one more workgroup per draft slot that selects the slot's keys meanwhile.
// Load hints of the statistics pass: non-temporal loads everywhere when the rows it streams
// exceed the Infinity Cache (the draw's re-read of row m then comes from HBM whatever the hint);
// for a large pass that fits, non-temporal loads on the draft rows of the later half of the
// slots and on the extra target row only. The first rejection is most often an early slot, so
// the draw mostly finds both of its rows in the cache, and the pass streams a third of its
// bytes at the faster non-temporal rate.
#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>

#include "api_common.hpp"
#include "row_keys.hpp"
#include "spec_common.hpp"

namespace sv {
namespace {

template <typename TIn>
__device__ __forceinline__ const TIn* slot_row(const TIn* tgt, const TIn* drf, int b, int r,
                                               int K, int V) {
  // rows 0..K are the request's target rows, rows K+1..2K its draft rows
  return r <= K ? tgt + (static_cast<size_t>(b) * (K + 1) + r) * static_cast<size_t>(V)
                : drf + (static_cast<size_t>(b) * K + (r - K - 1)) * static_cast<size_t>(V);
}

// log2(e) / T on the device, the same rounded value the host computes for a call's T
__device__ __forceinline__ float exp2_scale_dev(float T) {
  return static_cast<float>(1.4426950408889634074 / static_cast<double>(T));
}

// A thread's first maximum over chunk `cr` (elements visited in increasing token order), as
// (value, lowest id), then the workgroup's in thread 0.
template <typename TIn>
__device__ __forceinline__ void chunk_argmax(const TIn* row, const RowSpan& sp,
                                             const ChunkRange& cr, int V, float* s_v, int* s_i,
                                             float& M, int& I) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (cr.first && tid < sp.head) {
    bv = E::one(row, tid);
    bi = tid;
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
      for (int j = 0; j < N; ++j)
        if (t[j] > bv || (t[j] == bv && tok0 + j < bi)) {
          bv = t[j];
          bi = tok0 + j;
        }
    }
  }
  if (cr.last && tid < V - sp.tail) {
    const float v = E::one(row, sp.tail + tid);
    if (v > bv || (v == bv && sp.tail + tid < bi)) {
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

// Load hint of a launch of the statistics pass (uniform over the grid).
enum LoadHint : int {
  kHintCached = 0,       // ordinary loads: the rows stay in the Infinity Cache for the draw
  kHintStream = 1,       // non-temporal loads on every row
  kHintStreamDraft = 2,  // non-temporal loads on the draft rows of slots >= ceil(K/2) and on
                         // the extra target row
};

template <typename TIn, bool kKeys, bool kMixed, bool kPoint>
__global__ __launch_bounds__(kBlock) void sample_stats_kernel(
    const TIn* __restrict__ tgt, const TIn* __restrict__ drf, const int32_t* __restrict__ xtok,
    int K, int V, float c_call, int nchunk, int cv, float2* __restrict__ part,
    float* __restrict__ gath, uint64_t* __restrict__ clear, int nclear,
    float* __restrict__ key_wave_max, const float* __restrict__ temps,
    const int32_t* __restrict__ dlen, int nt) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  __shared__ float sm[kWaves], ss[kWaves];
  // the draw kernel that follows finds these words zero (nothing published yet)
  for (size_t gi = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x;
       gi < static_cast<size_t>(nclear); gi += static_cast<size_t>(gridDim.x) * kBlock)
    clear[gi] = 0ull;

  // point-mass drafts (kPoint) have no draft rows: only the K+1 target rows are streamed
  const int rows = kPoint ? K + 1 : 2 * K + 1;
  const int ch = blockIdx.x % nchunk;
  const int rb = blockIdx.x / nchunk;   // request-major (request, row) index
  const int r = rb % rows;
  const int b = rb / rows;
  if constexpr (kPoint) {
    // with draft lengths, target rows past n_b are never used (the draw reads row m <= n_b); a
    // length outside [0, K] is a row error and needs no row at all
    if (dlen != nullptr) {
      const int nb = dlen[b];
      if (nb < 0 || nb > K || r > nb) return;
    }
  }

  // per-request temperature (mixed batches): T_b = 0 is the greedy rule, which reads no draft
  // row and keeps each target chunk's (max, lowest id); an invalid T_b (a row error in the
  // draw) is treated the same way here
  float c = c_call;
  bool greedy = false;
  if constexpr (kMixed) {
    const float Tb = temps[b];
    greedy = !(Tb > 0.f);
    c = greedy ? 0.f : exp2_scale_dev(Tb);
    if (greedy && r > K) return;
  }

  const TIn* row = slot_row(tgt, drf, b, r, K, V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);

  if constexpr (kMixed) {
    if (greedy) {
      __shared__ int si[kWaves];
      float M;
      int I;
      chunk_argmax(row, sp, cr, V, sm, si, M, I);
      if (threadIdx.x == 0)
        part[static_cast<size_t>(rb) * nchunk + ch] = make_float2(M, __int_as_float(I));
      return;
    }
  }

  const int slot = r < K ? r : r - K - 1;

  float m, s, M, S;
  // The draw re-reads target row m (and draft row m below the extra row) right after this pass.
  // When the rows do not fit in the Infinity Cache, the re-read comes from HBM either way and
  // non-temporal loads only speed up the pass. When they fit, ordinary loads on every row keep
  // both re-read rows in the cache, which is best while the re-read is latency-bound (small
  // batches, mixed batches). For a large batch, the draft rows of the later slots (a first
  // rejection that late is the less likely) and the extra target row (whose re-read, on the
  // all-kept path, is one chunk) are streamed: that makes the pass faster, and row m is still
  // found in the cache for most requests. `nt` is uniform.
  const bool late_draft = r > K && r - K - 1 >= (K + 1) / 2;
  if (nt == kHintStream || (nt == kHintStreamDraft && (r == K || late_draft)))
    thread_chunk_stats<TIn, true, true>(row, sp, cr, V, c, m, s);
  else
    thread_chunk_stats<TIn, true, false>(row, sp, cr, V, c, m, s);
  // with outcome keys, a draft row's waves also keep their maxima (they bound where the row's
  // top tokens can be; the key merge re-reads only the waves that can hold one)
  float* wmax = (kKeys && r > K)
                    ? key_wave_max + ((static_cast<size_t>(b) * K + slot) * nchunk + ch) * kWaves
                    : nullptr;
  // The workgroup whose chunk holds the slot's draft token also reads that token's logit, so
  // the merge finds it without another dependent load. Rows 0..K-1 are target slots, K+1..2K
  // draft slots; row K (the extra target row) has no draft token. It is read once the chunk has
  // streamed (the chunk's lines were just fetched), so neither the draft token's load nor the
  // logit's delays the chunk's own loads.
  if (r != K && threadIdx.x == 0) {
    const int x = xtok[static_cast<size_t>(b) * K + slot];
    const int lo = cr.first ? 0 : sp.head + cr.vbeg * N;
    const int hi = cr.last ? V : sp.head + cr.vend * N;
    if (x >= lo && x < hi)
      gath[static_cast<size_t>(b) * 2 * K + (r < K ? slot : K + slot)] = E::one(row, x);
  }
  block_stats(m, s, c, sm, ss, M, S, wmax);
  if (threadIdx.x == 0) part[static_cast<size_t>(rb) * nchunk + ch] = make_float2(M, S);
}

// ------------------------------------------------------------------------------ draw
// Weights of the draw over row m: w = max(0, p - q) (residual, m < K) or w = p (bonus, m == K),
// with p = 2^((l - M_t) c - log2 S_t) and q likewise. `use_p` switches to w = p, the fallback when
// round-off leaves no residual mass.
// With a point-mass draft (kMask) the residual max(0, p - q) is p with the draft token `mask`
// removed (mask < 0: the bonus row, w = p).
template <typename TIn>
struct DrawRows {
  const TIn* t;
  const TIn* d;      // draft row m (unused for the bonus row)
  RowSpan sp;        // span of the target row; chunks follow it
  bool d_aligned;    // draft row has the same 16-byte phase, so vector loads line up
  bool resid;
  int mask;          // point-mass residual: the token whose weight is 0 (-1: none)
};

template <bool kMask, typename TIn>
__device__ __forceinline__ float weight_one(const DrawRows<TIn>& R, const ReqState& st, float c,
                                            int tok, bool use_p, float& p) {
  p = prob_exp2(Elem<TIn>::one(R.t, tok), st.M_t, c, st.ls_t);
  if constexpr (kMask) return (tok == R.mask && !use_p) ? 0.f : p;
  if (!R.resid || use_p) return p;
  const float q = prob_exp2(Elem<TIn>::one(R.d, tok), st.M_d, c, st.ls_d);
  return fmaxf(p - q, 0.f);
}

template <bool kMask, typename TIn>
__device__ __forceinline__ void weight_group(const DrawRows<TIn>& R, const ReqState& st, float c,
                                             const uint4& qt, const uint4& qd, int v, bool use_p,
                                             float (&w)[Elem<TIn>::N],
                                             float (&p)[Elem<TIn>::N]) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  float lt[N];
  E::unpack(qt, lt);
#pragma unroll
  for (int j = 0; j < N; ++j) p[j] = prob_exp2(lt[j], st.M_t, c, st.ls_t);
  if constexpr (kMask) {
    const int tok0 = R.sp.head + v * N;
#pragma unroll
    for (int j = 0; j < N; ++j) w[j] = (tok0 + j == R.mask && !use_p) ? 0.f : p[j];
    return;
  }
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
    w[j] = fmaxf(p[j] - prob_exp2(ld[j], st.M_d, c, st.ls_d), 0.f);
}

template <typename TIn>
__device__ __forceinline__ void load_pair(const DrawRows<TIn>& R, int v, bool has, uint4& qt,
                                          uint4& qd) {
  const uint4* tv = reinterpret_cast<const uint4*>(R.t + R.sp.head);
  const uint4* dv = reinterpret_cast<const uint4*>(R.d + R.sp.head);
  qt = has ? load_global(tv, v) : neg_inf_vec<TIn>();
  qd = (has && R.resid && R.d_aligned) ? load_global(dv, v) : neg_inf_vec<TIn>();
}

// The elements a thread of the draw owns, in token order: the scalar head (thread 0 of chunk 0),
// its kDrawVecs adjacent vectors, then the scalar tail (the thread holding the row's last
// vector, or the head's owner when the row has no whole vector). Every thread's elements are
// contiguous in token order, so the thread order of the chunks is token order.
struct ThreadElems {
  int nh;      // head elements [0, nh)
  int v0, nv;  // vectors [v0, v0 + nv)
  int nt;      // tail elements [tail0, tail0 + nt)
  int tail0;
};

__device__ __forceinline__ ThreadElems thread_elems(const RowSpan& sp, int V, int nchunk, int cv,
                                                    int ch, int th) {
  const ChunkRange cr = chunk_range(sp, ch, nchunk, cv);
  ThreadElems e;
  e.v0 = cr.vbeg + th * kDrawVecs;
  e.nv = max(0, min(kDrawVecs, cr.vend - e.v0));
  e.nh = (ch == 0 && th == 0) ? sp.head : 0;
  int tch = 0, tth = 0;
  if (sp.nvec > 0) {
    const int lv = sp.nvec - 1;
    tch = lv / cv;
    tth = (lv - tch * cv) / kDrawVecs;
  }
  e.nt = (ch == tch && th == tth) ? V - sp.tail : 0;
  e.tail0 = sp.tail;
  return e;
}

// One thread's draw mass ws (sum of w) and target mass ps (sum of p), summed in token order;
// `qt`/`qd` receive its vectors. Deterministic: the owner and any helper get the same bits.
template <bool kMask, typename TIn>
__device__ __forceinline__ void thread_mass(const DrawRows<TIn>& R, const ReqState& st, float c,
                                            int V, const ThreadElems& el, uint4 (&qt)[kDrawVecs],
                                            uint4 (&qd)[kDrawVecs], float& ws, float& ps) {
  constexpr int N = Elem<TIn>::N;
#pragma unroll
  for (int i = 0; i < kDrawVecs; ++i) load_pair(R, el.v0 + i, i < el.nv, qt[i], qd[i]);
  ws = 0.f;
  ps = 0.f;
  float p;
  for (int e = 0; e < el.nh; ++e) {
    ws += weight_one<kMask>(R, st, c, e, false, p);
    ps += p;
  }
#pragma unroll
  for (int i = 0; i < kDrawVecs; ++i) {
    if (i < el.nv) {
      float wv[N], pv[N];
      weight_group<kMask>(R, st, c, qt[i], qd[i], el.v0 + i, false, wv, pv);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        ws += wv[j];
        ps += pv[j];
      }
    }
  }
  for (int e = 0; e < el.nt; ++e) {
    ws += weight_one<kMask>(R, st, c, el.tail0 + e, false, p);
    ps += p;
  }
}

// Chunk masses (R, P) in float64 from the threads' (ws, ps): wave butterflies, then the four
// wave totals in order. Every thread returns the same bits.
__device__ __forceinline__ void chunk_mass(float ws, float ps, double (*s_red)[kWaves],
                                           double& R, double& P) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const double rw = group_reduce(static_cast<double>(ws), kWave, OpAdd{});
  const double pw = group_reduce(static_cast<double>(ps), kWave, OpAdd{});
  if (lane == 0) {
    s_red[0][w] = rw;
    s_red[1][w] = pw;
  }
  __syncthreads();
  R = 0.0;
  P = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    R += s_red[0][i];
    P += s_red[1][i];
  }
  __syncthreads();   // s_red is reused
}

constexpr uint64_t kWrittenBit = 1ull << 63;   // sign bit of a non-negative float64 mass

// Reads a published (R, P) pair, re-polling at most `polls` times; false if it is not there yet.
__device__ __forceinline__ bool poll_mass(const uint64_t* p, int polls, double& R, double& P) {
  uint64_t a = load_coherent(p), b = load_coherent(p + 1);
  while (((a & b) & kWrittenBit) == 0ull) {
    if (polls-- <= 0) return false;
    __builtin_amdgcn_s_sleep(2);
    if ((a & kWrittenBit) == 0ull) a = load_coherent(p);
    if ((b & kWrittenBit) == 0ull) b = load_coherent(p + 1);
  }
  R = bits_d(a & ~kWrittenBit);
  P = bits_d(b & ~kWrittenBit);
  return true;
}

// most draw chunks a row of V <= SPEC_MAX_V elements can have (f32 rows: 4 elements per vector)
constexpr int kMaxDrawChunks = (SPEC_MAX_V / 4 + kBlock * kDrawVecs - 1) / (kBlock * kDrawVecs);

// Outcome keys computed alongside the verification: where the statistics pass left the wave
// maxima and where the keys go.
struct KeyArgs {
  int pick;            // tokens looked for per slot: F, or F + 1 with the draft token skipped
  int F;               // keys written per slot
  int exclude;         // skip the draft token
  int cv_s;            // statistics chunk size (vectors)
  const float* wave_max;   // [B,K,nchunk_s,4]: the statistics pass's wave maxima of draft rows
  int32_t* out_keys;       // [B,K,F]
  float* out_prob;         // [B,K,F] or null
};

// A row's (max, sum) from its n chunk partials pr[0..n), merged by an aligned group of W lanes
// (W a power of two; lane i of the group holds chunks i, i + W, ...): every lane of the group
// gets the same bits, wherever the group sits in the wave. has = false (a group without a row)
// gives (-inf, 0).
constexpr int kMergeHeld = 4;   // chunks a lane keeps in registers between the merge's two passes

// `rd(j)` returns chunk j's (max, sum).
template <typename Rd>
__device__ __forceinline__ void merge_row_stats_rd(Rd rd, bool has, int n, int W, int i, float c,
                                                   float& Mr, double& Sr) {
  constexpr int kHeld = kMergeHeld;
  float hm[kHeld], hs[kHeld];
  float lm = -INFINITY;
#pragma unroll
  for (int h = 0; h < kHeld; ++h) {
    const int j = i + h * W;
    const float2 q = (has && j < n) ? rd(j) : make_float2(-INFINITY, 0.f);
    hm[h] = q.x;
    hs[h] = q.y;
    lm = fmaxf(lm, hm[h]);
  }
  if (has)
    for (int j = i + kHeld * W; j < n; j += W) lm = fmaxf(lm, rd(j).x);
  Mr = group_reduce(lm, W, OpMax{});
  double ls = 0.0;
#pragma unroll
  for (int h = 0; h < kHeld; ++h)
    if (hm[h] > -INFINITY) ls += static_cast<double>(hs[h]) * rel_exp2(hm[h], Mr, c);
  if (has)
    for (int j = i + kHeld * W; j < n; j += W) {
      const float2 q = rd(j);
      if (q.x > -INFINITY) ls += static_cast<double>(q.y) * rel_exp2(q.x, Mr, c);
    }
  Sr = group_reduce(ls, W, OpAdd{});
}

__device__ __forceinline__ void merge_row_stats(const float2* pr, bool has, int n, int W, int i,
                                                float c, float& Mr, double& Sr) {
  merge_row_stats_rd([pr](int j) { return load_f2(pr + j); }, has, n, W, i, c, Mr, Sr);
}

// The group width the merges use for `rows` rows of n chunks: the widest power of two (at most
// 64, one chunk per lane) with which the block's waves take every row in one pass, but not so
// narrow that a lane would hold more than kMergeHeld chunks (then the rows take several passes).
// One pass issues every partial load at once; each pass costs a round trip.
__device__ __forceinline__ int merge_width(int n, int rows) {
  int lo = 1;
  while (lo * kMergeHeld < n && lo < kWave) lo <<= 1;
  int W = 1;
  while (W < n && W < kWave) W <<= 1;
  while (W > lo && kWaves * (kWave / W) < rows) W >>= 1;
  return W;
}

// ------------------------------------------------------------------------------ draw phases
// LDS of a workgroup drawing one chunk of row m.
struct DrawShared {
  double s_red[2][kWaves];
  double2 s_cm[kMaxDrawChunks];            // every chunk's (residual mass, target mass)
  int s_first[kWaves];
  uint32_t s_raw[2][4 * kDrawVecs];        // one thread's target and draft vectors
  int s_cs, s_usep, s_fallback;
  double s_cb, s_t;
  float row_m[2 * SPEC_MAX_K + 1];
  double row_s[2 * SPEC_MAX_K + 1];
  ReqState s_st;
};

// Chunk masses published with the sign bit of each float64 word as the "written" flag; the
// words are zeroed by the statistics kernel of the same call, before the draw kernel starts.
struct FlaggedMasses {
  uint64_t* cm;   // [nchunk][2] of one request
  __device__ void publish(int j, double R, double P) const {
    store_coherent(&cm[2 * j], dbits(R) | kWrittenBit);
    store_coherent(&cm[2 * j + 1], dbits(P) | kWrittenBit);
  }
  __device__ bool poll(int j, int polls, double& R, double& P) const {
    return poll_mass(&cm[2 * j], polls, R, P);
  }
};

// Wave 0 of a draw workgroup of request b, from the merged row statistics in sh.row_m/row_s and
// each lane's slot (lane k < nb: draft token xk, uniform uk, gathered target and draft logits
// lt, ld): every slot's acceptance ratio, the first rejection m by ballot; chunk 0 writes tau,
// kv, the kept tokens, p and q. The draw's state goes to sh.s_st (m = -1 for a row error).
template <bool kPoint>
__device__ __forceinline__ void decide_slots(int b, int ch, int K, int V, float c, int nb,
                                             bool nb_bad, bool valid, int xk, float uk, float lt,
                                             float ld, int kv0, DrawShared& sh,
                                             int32_t* __restrict__ out_tok,
                                             int32_t* __restrict__ out_tau,
                                             int32_t* __restrict__ out_kv,
                                             float* __restrict__ out_p,
                                             float* __restrict__ out_q) {
  const int lane = threadIdx.x & (kWave - 1);
  // a draft token must be a token the draft could have sampled
  const bool bad = valid && (xk < 0 || xk >= V || (!kPoint && ld == -INFINITY));
  bool keep = true;
  float pk = 0.f, qk = 0.f;
  if (valid && !bad) {
    // log2 p_k(x_k) = (l - M) c - log2 S of the target row, with l - M the draft token's gap
    // below the row maximum; log2 q_k(x_k) likewise (0 for a point-mass draft), and
    // log2(p/q) = (g_t - g_d) c + log2 S_d - log2 S_t from the two gaps, which stays finite (or
    // -inf for a masked target logit) at every temperature. In float32 and the log domain:
    // accurate to ~3e-6 relative in p, q and the ratio (inside the 1e-5 margin that flags a
    // decision as a near-tie), and neither p nor q can underflow the ratio (a float64
    // evaluation cost ~1 us on every draw workgroup's critical path). S >= 1: the row's maximum
    // contributes 2^0.
    const float gt = lt - sh.row_m[lane];
    const float lst = __builtin_amdgcn_logf(static_cast<float>(sh.row_s[lane]));
    const float lp = gt * c - lst;
    float lr = lp;   // log2 (p/q)
    if constexpr (!kPoint) {
      const float gd = ld - sh.row_m[K + 1 + lane];
      const float lsd = __builtin_amdgcn_logf(static_cast<float>(sh.row_s[K + 1 + lane]));
      qk = fast_exp2(gd * c - lsd);
      lr = (gt - gd) * c + (lsd - lst);
    } else {
      qk = 1.f;
    }
    pk = fast_exp2(lp);
    // kept iff u < min(1, p/q): p >= q is kept for every u in [0,1)
    keep = lr >= 0.f || uk < fast_exp2(lr);
  }
  const bool err = nb_bad || __ballot(bad) != 0ull;
  const unsigned long long rej = __ballot(valid && !keep);
  const int mm = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : nb;
  const int xm = __shfl(xk, mm < nb ? mm : 0, kWave);   // the rejected draft token
  if (ch == 0) {   // one workgroup of the request writes everything but the drawn token
    if (lane < K) {   // slots past the request's drafts report NaN
      const size_t o = static_cast<size_t>(b) * K + lane;
      if (out_p) out_p[o] = (err || !valid) ? NAN : pk;
      if (out_q) out_q[o] = (err || !valid) ? NAN : qk;
    }
    for (int j = lane; j <= K; j += kWave)
      if (err || j != mm)
        out_tok[static_cast<size_t>(b) * (K + 1) + j] = (!err && j < mm) ? xk : -1;
    if (lane == 0) {
      out_tau[b] = err ? -1 : mm + 1;
      if (out_kv) out_kv[b] = err ? kv0 : kv0 + mm + 1;
    }
  }
  if (lane == 0) {
    ReqState st;
    st.m = err ? -1 : mm;
    st.xm = (kPoint && mm < nb) ? xm : -1;
    st.M_t = sh.row_m[mm];
    st.ls_t = __builtin_amdgcn_logf(static_cast<float>(sh.row_s[mm]));
    st.M_d = (!kPoint && mm < K) ? sh.row_m[K + 1 + mm] : 0.f;
    st.ls_d = (!kPoint && mm < K) ? __builtin_amdgcn_logf(static_cast<float>(sh.row_s[K + 1 + mm]))
                                  : 0.f;
    sh.s_st = st;
  }
}

// Rows m of request b as the draw reads them.
template <typename TIn>
__device__ __forceinline__ DrawRows<TIn> draw_rows(const TIn* tgt, const TIn* drf, int b, int K,
                                                   int V, const ReqState& st, bool point) {
  DrawRows<TIn> R;
  R.resid = !point && st.m < K;
  R.mask = st.xm;
  R.t = tgt + (static_cast<size_t>(b) * (K + 1) + st.m) * static_cast<size_t>(V);
  R.d = R.resid ? drf + (static_cast<size_t>(b) * K + st.m) * static_cast<size_t>(V) : R.t;
  R.sp = row_span(R.t, V);
  R.d_aligned = row_span(R.d, V).head == R.sp.head;
  return R;
}

// The chunk holding u*Z, as every lane of a wave finds it once sh.s_cm holds every chunk's
// (residual mass, target mass): float64 prefix scan over the chunks (lane l takes a contiguous run
// of them), total Z, threshold t = u*Z, then the chunk whose running mass passes t. Every wave
// that runs it gets the same bits, in registers.
struct ChunkPick {
  int cs;          // the chunk holding u*Z
  bool usep;       // no residual mass left by round-off: the draw takes p
  bool fallback;   // round-off: no chunk's running mass passed t (cs is the last of positive mass)
  double cb;       // mass of the chunks before cs
  double t;        // u*Z
};

__device__ __forceinline__ ChunkPick pick_chunk(int nchunk, float u_draw, const DrawShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (nchunk + kWave - 1) / kWave;
  const int j0 = min(lane * per, nchunk), j1 = min(j0 + per, nchunk);
  double rl = 0.0, pl = 0.0;
  int lr = -1, lp = -1;
  for (int j = j0; j < j1; ++j) {
    const double2 m2 = sh.s_cm[j];
    rl += m2.x;
    pl += m2.y;
    if (m2.x > 0.0) lr = j;
    if (m2.y > 0.0) lp = j;
  }
  const double ri = wave_scan_incl(rl), pi = wave_scan_incl(pl);
  const double zr = readlane_f64(ri, kWave - 1), zp = readlane_f64(pi, kWave - 1);
  ChunkPick f;
  f.usep = !(zr > 0.0);
  const double Z = f.usep ? zp : zr;
  f.t = static_cast<double>(u_draw) * Z;
  const double incl = f.usep ? pi : ri;
  const double excl = wave_shift_up1(incl);
  const unsigned long long cross = __ballot(incl > f.t);
  const int last_pos = group_reduce(f.usep ? lp : lr, kWave, OpMax{});
  if (cross) {
    // lane L's run holds the crossing; every lane walks its own run, lane L's result is taken
    const int L = __ffsll(static_cast<long long>(cross)) - 1;
    double cum = excl;
    int cs = -1, lastp = -1;
    for (int j = j0; j < j1; ++j) {
      const double mj = f.usep ? sh.s_cm[j].y : sh.s_cm[j].x;
      if (mj > 0.0) lastp = j;
      if (cum + mj > f.t) {
        cs = j;
        break;
      }
      cum += mj;
    }
    f.cs = __builtin_amdgcn_readlane(cs >= 0 ? cs : max(lastp, 0), L);
    f.fallback = __builtin_amdgcn_readlane(cs >= 0 ? 0 : 1, L) != 0;
    f.cb = readlane_f64(cum, L);
  } else {   // round-off: the last chunk of positive weight
    f.cs = max(last_pos, 0);
    f.fallback = true;
    f.cb = 0.0;
  }
  return f;
}

// Wave 0's pick_chunk, left in sh (s_cs, s_usep, s_fallback, s_cb, s_t) for the workgroup.
__device__ __forceinline__ void find_chunk(int nchunk, float u_draw, DrawShared& sh) {
  const ChunkPick f = pick_chunk(nchunk, u_draw, sh);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.s_cs = f.cs;
    sh.s_fallback = f.fallback ? 1 : 0;
    sh.s_cb = f.cb;
    sh.s_usep = f.usep ? 1 : 0;
    sh.s_t = f.t;
  }
}

// The block-level part of the search that does not depend on which chunk holds u*Z: every
// thread's inclusive scan of its draw mass within its wave, the wave totals and the last thread
// of positive mass. Taken right after a workgroup publishes its chunk's masses, it overlaps the
// wait for the other chunks' masses; search_in_chunk then adds the same terms in the same order
// as when it takes the scan itself, so the bits are the same.
struct ScanPrep {
  double wi;
  double tot[kWaves];   // every wave's total (its last lane's inclusive sum)
  double top[kWaves];   // every wave's largest inclusive sum
  int last_thr;
};

__device__ __forceinline__ ScanPrep scan_prep(float mine, DrawShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  ScanPrep p;
  p.wi = wave_scan_incl(static_cast<double>(mine));
  if (lane == kWave - 1) sh.s_red[0][w] = p.wi;
  const double top = group_reduce(p.wi, kWave, OpMax{});
  if (lane == 0) sh.s_red[1][w] = top;
  const int lpos = group_reduce(mine > 0.f ? tid : -1, kWave, OpMax{});
  if (lane == 0) sh.s_first[w] = lpos;
  __syncthreads();
  // the same in every lane: kept in scalar registers
  int last = -1;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    p.tot[i] = readlane_f64(sh.s_red[0][i], 0);
    p.top[i] = readlane_f64(sh.s_red[1][i], 0);
    last = max(last, sh.s_first[i]);
  }
  p.last_thr = __builtin_amdgcn_readfirstlane(last);
  return p;   // s_red and s_first are rewritten only after the caller's next barrier
}

// One wave, once thread `first` of chunk `ch` has left its vectors in sh.s_raw and its prefix
// mass in sh.s_cb: one element of that thread per lane (at most 7 + 32 + 7 for bf16), in token
// order, weights as in its mass, float64 prefix scan, the first element past t (with walk_fb, the
// last element of positive weight), written to *out_y.
template <typename TIn, bool kPoint>
__device__ __forceinline__ void token_in_thread(const DrawRows<TIn>& R, const ReqState& st,
                                                float c, int V, int nchunk, int cv, int ch,
                                                int first, bool use_p, bool walk_fb, double t,
                                                const DrawShared& sh,
                                                int32_t* __restrict__ out_y) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  const int lane = threadIdx.x & (kWave - 1);
  const ThreadElems fe = thread_elems(R.sp, V, nchunk, cv, ch, first);
  const int nvel = fe.nv * N;
  const bool has = lane < fe.nh + nvel + fe.nt;
  int tok = 0;
  float lt = -INFINITY, ld = -INFINITY;
  if (has) {
    if (lane < fe.nh || lane >= fe.nh + nvel) {   // scalar head or tail element
      tok = lane < fe.nh ? lane : fe.tail0 + (lane - fe.nh - nvel);
      lt = E::one(R.t, tok);
      if (R.resid) ld = E::one(R.d, tok);
    } else {
      const int k = lane - fe.nh, i = k / N, e = k % N;
      tok = R.sp.head + (fe.v0 + i) * N + e;
      lt = E::from_words(&sh.s_raw[0][4 * i], e);
      if (R.resid) ld = R.d_aligned ? E::from_words(&sh.s_raw[1][4 * i], e) : E::one(R.d, tok);
    }
  }
  float we = 0.f;
  if (has) {
    const float p = prob_exp2(lt, st.M_t, c, st.ls_t);
    if constexpr (kPoint)
      we = (tok == R.mask && !use_p) ? 0.f : p;
    else
      we = (!R.resid || use_p) ? p : fmaxf(p - prob_exp2(ld, st.M_d, c, st.ls_d), 0.f);
  }
  const double cum = sh.s_cb + wave_scan_incl(static_cast<double>(we));
  const unsigned long long pos = __ballot(we > 0.f);
  const unsigned long long hit = walk_fb ? 0ull : __ballot(we > 0.f && cum > t);
  int y;
  if (hit) y = __shfl(tok, __ffsll(static_cast<long long>(hit)) - 1, kWave);
  else if (pos) y = __shfl(tok, 63 - __clzll(static_cast<long long>(pos)), kWave);
  else y = 0;   // no positive weight at all: only for rows without a finite logit
  if (lane == 0) *out_y = y;
}

// The workgroup of the chunk holding u*Z (chunk `ch`, its threads' masses ws/ps and elements el
// as thread_mass gave them): the thread holding it (block prefix scan of the thread masses), then
// the token among that thread's elements, which it hands to wave 0 through LDS; writes the token
// to *out_y. Called by the whole workgroup. With kHeld the caller kept every thread's vectors in
// registers across the mass exchange (32 more registers per thread) and passes them, and `prep`
// (if given) is the scan it took meanwhile; otherwise the vectors are read again here (from the
// cache). With kRecompute (a workgroup that published several chunks and kept none of their
// thread masses) ws and ps are computed again from the vectors read here: thread_mass gives the
// same bits.
template <typename TIn, bool kPoint, bool kRecompute = false, bool kHeld = false>
__device__ __forceinline__ void search_in_chunk(const DrawRows<TIn>& R, const ReqState& st,
                                                float c, int V, int nchunk, int cv, int ch,
                                                const ThreadElems& el, float ws, float ps,
                                                DrawShared& sh, int32_t* __restrict__ out_y,
                                                const uint4* held_t = nullptr,
                                                const uint4* held_d = nullptr,
                                                const ScanPrep* prep = nullptr) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  // every thread reads its vectors again now (cache hits), so the one that turns out to hold
  // u*Z has them when the block scan below has named it (kHeld: the caller kept them)
  uint4 qt[kDrawVecs], qd[kDrawVecs];
  if constexpr (kHeld) {
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      qt[i] = held_t[i];
      qd[i] = held_d[i];
    }
  } else if constexpr (kRecompute) {
    thread_mass<kPoint>(R, st, c, V, el, qt, qd, ws, ps);
  } else {
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) load_pair(R, el.v0 + i, i < el.nv, qt[i], qd[i]);
  }
  const bool use_p = sh.s_usep != 0;
  const bool fb = sh.s_fallback != 0;
  const double t = sh.s_t;
  const float mine = use_p ? ps : ws;
  double wi, off = sh.s_cb;
  int last_thr = -1;
  if (prep != nullptr && !use_p) {   // uniform: the scan of ws was taken during the exchange
    wi = prep->wi;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
      if (i < w) off += prep->tot[i];
    last_thr = prep->last_thr;
  } else {
    wi = wave_scan_incl(static_cast<double>(mine));
    if (lane == kWave - 1) sh.s_red[0][w] = wi;
    const int lpos = group_reduce(mine > 0.f ? tid : -1, kWave, OpMax{});
    if (lane == 0) sh.s_first[w] = lpos;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      if (i < w) off += sh.s_red[0][i];
      last_thr = max(last_thr, sh.s_first[i]);
    }
  }
  const double incl = off + wi;
  const double excl = off + wave_shift_up1(wi);
  const unsigned long long cross = fb ? 0ull : __ballot(incl > t);
  __syncthreads();   // s_first is rewritten
  if (lane == 0)
    sh.s_first[w] = cross ? w * kWave + __ffsll(static_cast<long long>(cross)) - 1 : -1;
  __syncthreads();
  int first = -1;
#pragma unroll
  for (int i = kWaves - 1; i >= 0; --i)
    if (sh.s_first[i] >= 0) first = sh.s_first[i];
  const bool walk_fb = first < 0;   // round-off (or fallback): the last thread of positive mass
  if (walk_fb) first = max(last_thr, 0);
  if (tid == first) {   // hand this thread's vectors and prefix to wave 0
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      sh.s_raw[0][4 * i] = qt[i].x;
      sh.s_raw[0][4 * i + 1] = qt[i].y;
      sh.s_raw[0][4 * i + 2] = qt[i].z;
      sh.s_raw[0][4 * i + 3] = qt[i].w;
      sh.s_raw[1][4 * i] = qd[i].x;
      sh.s_raw[1][4 * i + 1] = qd[i].y;
      sh.s_raw[1][4 * i + 2] = qd[i].z;
      sh.s_raw[1][4 * i + 3] = qd[i].w;
    }
    sh.s_cb = excl;
  }
  __syncthreads();

  if (w == 0) token_in_thread<TIn, kPoint>(R, st, c, V, nchunk, cv, ch, first, use_p, walk_fb, t,
                                          sh, out_y);
}

// The search of search_in_chunk for a workgroup that kept its vectors and took its scan during
// the exchange (prep), when the draw takes the residual or bonus weights (not the round-off
// fallback to p): no workgroup barrier. The wave totals and each wave's largest inclusive sum
// tell every wave, with the same additions in the same order as the block scan, which wave's
// ballot would find the first thread past t; that wave alone goes on, its lane of that thread
// hands its vectors over through LDS (one wave: no barrier), and it finds the token.
template <typename TIn, bool kPoint>
__device__ __forceinline__ void search_in_wave(const DrawRows<TIn>& R, const ReqState& st,
                                               float c, int V, int nchunk, int cv, int ch,
                                               const ChunkPick& f, const ScanPrep& prep,
                                               const uint4 (&qt)[kDrawVecs],
                                               const uint4 (&qd)[kDrawVecs], DrawShared& sh,
                                               int32_t* __restrict__ out_y) {
  const int tid = threadIdx.x, w = tid / kWave;
  const double t = f.t;
  int owner = -1;        // the first wave with a thread past t
  double off_w = f.cb;   // this wave's offset, as the block scan forms it
  {
    double off = f.cb;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      if (i == w) off_w = off;
      if (owner < 0 && !f.fallback && off + prep.top[i] > t) owner = i;
      off += prep.tot[i];
    }
  }
  const bool walk_fb = owner < 0;   // round-off (or fallback): the last thread of positive mass
  const int first_w = walk_fb ? max(prep.last_thr, 0) / kWave : owner;
  if (w != first_w) return;
  const double incl = off_w + prep.wi;
  const double excl = off_w + wave_shift_up1(prep.wi);
  const unsigned long long cross = __ballot(incl > t);
  const int first = walk_fb ? max(prep.last_thr, 0)
                            : w * kWave + __ffsll(static_cast<long long>(cross)) - 1;
  if (tid == first) {   // hand this thread's vectors and prefix to its wave
#pragma unroll
    for (int i = 0; i < kDrawVecs; ++i) {
      sh.s_raw[0][4 * i] = qt[i].x;
      sh.s_raw[0][4 * i + 1] = qt[i].y;
      sh.s_raw[0][4 * i + 2] = qt[i].z;
      sh.s_raw[0][4 * i + 3] = qt[i].w;
      sh.s_raw[1][4 * i] = qd[i].x;
      sh.s_raw[1][4 * i + 1] = qd[i].y;
      sh.s_raw[1][4 * i + 2] = qd[i].z;
      sh.s_raw[1][4 * i + 3] = qd[i].w;
    }
    sh.s_cb = excl;
  }
  __builtin_amdgcn_wave_barrier();
  token_in_thread<TIn, kPoint>(R, st, c, V, nchunk, cv, ch, first, false, walk_fb, t, sh, out_y);
}

// Every chunk mass marked missing in sh.s_cm (R < 0: not published within the poll budget),
// computed by this workgroup: the same bits the chunk's own workgroup publishes. Called by the
// whole workgroup after a barrier.
template <typename TIn, bool kPoint>
__device__ __forceinline__ void help_missing_masses(const DrawRows<TIn>& R, const ReqState& st,
                                                 float c, int V, int nchunk, int cv,
                                                 DrawShared& sh) {
  const int tid = threadIdx.x;
  for (int j = 0; j < nchunk; ++j) {
    if (!(sh.s_cm[j].x < 0.0)) continue;   // uniform: read after a barrier
    uint4 ht[kDrawVecs], hd[kDrawVecs];
    float hw, hp;
    thread_mass<kPoint>(R, st, c, V, thread_elems(R.sp, V, nchunk, cv, j, tid), ht, hd, hw, hp);
    double hr, hq;
    chunk_mass(hw, hp, sh.s_red, hr, hq);
    if (tid == 0) sh.s_cm[j] = make_double2(hr, hq);
    __syncthreads();
  }
}

// Chunks of kBlock * kDrawVecs vectors (see draw_plan); each workgroup takes `group` consecutive
// chunks of its request (draw_group: one, unless the chunks would not all be resident at once).
// kGroups = false is the one-chunk instance (group is then 1 and folds away).
// cm holds the published (R, P) of every chunk, [b][ch][2] words, zeroed by the statistics
// kernel of the same call.
template <typename TIn, bool kKeys, bool kMixed, bool kPoint, bool kGroups>
__global__ __launch_bounds__(kBlock) void sample_draw_kernel(
    const TIn* __restrict__ tgt, const TIn* __restrict__ drf, const int32_t* __restrict__ xtok,
    const float* __restrict__ uni, const int32_t* __restrict__ kv_in, int K, int V, float c_call,
    int nchunk_s, const float2* __restrict__ part_s, const float* __restrict__ gath,
    int nchunk, int cv, int aligned, int group, uint64_t* __restrict__ cm, int wait_polls,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_tau, int32_t* __restrict__ out_kv,
    float* __restrict__ out_p, float* __restrict__ out_q, KeyArgs ka,
    const float* __restrict__ temps, const int32_t* __restrict__ dlen, int n_draw) {
  __shared__ DrawShared sh;

  if constexpr (kKeys) {
    // ---- the workgroups past the draw's select one draft slot's outcome keys each, alongside
    // the draw (they wait on nothing). The slot's row statistics are merged by wave 0 exactly as
    // the draw merges them (same group width, same lanes' chunks), so q_k(key) uses the same
    // (M, S) bits as out_q.
    if (static_cast<int>(blockIdx.x) >= n_draw) {
      const size_t bk = blockIdx.x - n_draw;   // b * K + k
      const int kb = static_cast<int>(bk / K), kk = static_cast<int>(bk % K);
      const int lane = threadIdx.x & (kWave - 1);
      const int xk = ka.exclude ? xtok[bk] : -1;
      const float2* pr = part_s + (static_cast<size_t>(kb) * (2 * K + 1) + K + 1 + kk) * nchunk_s;
      const int Wk = merge_width(nchunk_s, 2 * K + 1);   // as the draw's merge below
      auto row_stat = [&]() {
        float Mr;
        double Sr;
        merge_row_stats(pr, lane < Wk, nchunk_s, Wk, lane % Wk, c_call, Mr, Sr);
        return RowStat{readlane_f32(Mr, 0), 0.f, readlane_f64(Sr, 0)};
      };
      select_keys<TIn, kWaves, false>(drf + bk * static_cast<size_t>(V), V, nchunk_s, ka.cv_s,
                                      ka.wave_max + bk * static_cast<size_t>(nchunk_s * kWaves),
                                      ka.pick, ka.F, xk, row_stat, c_call,
                                      ka.out_keys + bk * ka.F,
                                      ka.out_prob ? ka.out_prob + bk * ka.F : nullptr);
      return;
    }
  }

  const int grp = kGroups ? group : 1;
  const int nq = kGroups ? (nchunk + grp - 1) / grp : nchunk;   // workgroups per request
  const int b = blockIdx.x / nq;
  const int c0 = static_cast<int>(blockIdx.x % nq) * grp;   // this workgroup's chunks [c0, c1)
  const int c1 = kGroups ? min(c0 + grp, nchunk) : c0 + 1;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int rows = kPoint ? K + 1 : 2 * K + 1;

  // drafts in this request: K, or (point-mass drafts with lengths) the first dlen[b] slots; a
  // length outside [0, K] is a row error
  int nb = K;
  bool nb_bad = false;
  if constexpr (kPoint) {
    if (dlen != nullptr) {
      nb = dlen[b];
      nb_bad = nb < 0 || nb > K;
      if (nb_bad) nb = 0;
    }
  }

  float c = c_call;
  if constexpr (kMixed) {
    // ---- per-request temperature: T_b = 0 takes the greedy rule on the (max, lowest id) chunk
    // partials of the target rows; a T_b that is negative, not finite, or too small for log2(e)/T
    // to be finite is a row error
    __shared__ int row_g[SPEC_MAX_K + 1];
    const float Tb = temps[b];
    const bool greedy = Tb == 0.f;
    const float cc = Tb > 0.f ? exp2_scale_dev(Tb) : 0.f;
    const bool t_ok = greedy || (Tb > 0.f && isfinite(Tb) && isfinite(cc));
    c = cc;
    if (greedy || !t_ok) {
      if (c0 != 0) return;   // one workgroup of the request does all of it
      // wave 0's draft tokens are loaded first, so their latency passes during the merges
      const bool valid = lane < K;
      const int xk = (w == 0 && valid) ? xtok[static_cast<size_t>(b) * K + lane] : 0;
      if (t_ok) {
        // rows in groups of G lanes (nchunk_s rounded up to a power of two, at most a wave), so
        // every partial of up to 4 * 64 / G rows is loaded at once; the (max, lowest id) merge
        // gives the same pair in any order
        int G = 1;
        while (G < nchunk_s && G < kWave) G <<= 1;
        const int per_wave = kWave / G, g = lane / G, gi = lane % G;
        for (int base = 0; base <= K; base += kWaves * per_wave) {
          const int rr = base + w * per_wave + g;
          float v = -INFINITY;
          int i = 0x7fffffff;
          if (rr <= K) {
            const float2* pr = part_s + (static_cast<size_t>(b) * rows + rr) * nchunk_s;
            for (int j = gi; j < nchunk_s; j += G) {
              const float2 q = load_f2(pr + j);
              if (better(q.x, __float_as_int(q.y), v, i)) {
                v = q.x;
                i = __float_as_int(q.y);
              }
            }
          }
          for (int off = G / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(v, off, kWave);
            const int oi = __shfl_xor(i, off, kWave);
            if (better(ov, oi, v, i)) {
              v = ov;
              i = oi;
            }
          }
          // a row whose logits are all -inf keeps no index: its first token is the lowest id
          if (gi == 0 && rr <= K) row_g[rr] = i == 0x7fffffff ? 0 : i;
        }
      }
      __syncthreads();
      if (w != 0) return;
      const bool err = __ballot(!t_ok || (valid && (xk < 0 || xk >= V))) != 0ull;
      const unsigned long long miss = __ballot(!err && valid && xk != row_g[valid ? lane : 0]);
      const int mm = miss ? __ffsll(static_cast<long long>(miss)) - 1 : K;
      if (valid) {   // at temperature zero p_k(x_k) is 1 for the target's top choice, else 0
        const size_t o = static_cast<size_t>(b) * K + lane;
        if (out_p) out_p[o] = err ? NAN : (xk == row_g[lane] ? 1.f : 0.f);
        if (out_q) out_q[o] = err ? NAN : 1.f;
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
      }
      return;
    }
  }

  // ---- merge the statistics pass of request b (every workgroup of b does the same, bit for
  // bit): row (max, sum) in fp32/fp64, slot acceptance ratios, first rejection by ballot
  {
    const bool valid = w == 0 && lane < nb;
    int xk = 0;
    float lt = 0.f, ld = 0.f, uk = 0.f;
    if (valid) {
      xk = xtok[static_cast<size_t>(b) * K + lane];
      uk = uni[static_cast<size_t>(b) * (K + 1) + lane];
      lt = gath[static_cast<size_t>(b) * 2 * K + lane];
      if constexpr (!kPoint) ld = gath[static_cast<size_t>(b) * 2 * K + K + lane];
    }
    const int kv0 = (c0 == 0 && tid == 0 && kv_in) ? kv_in[b] : 0;
    // Rows are merged in groups of W lanes (merge_width), 64/W rows per wave, so one pass over
    // the block issues every partial load at once. Lanes past nchunk_s (or past the last row)
    // carry (-inf, 0).
    const int W = merge_width(nchunk_s, rows);
    const int per_wave = kWave / W, g = lane / W, i = lane % W;
    for (int base = 0; base < rows; base += kWaves * per_wave) {
      const int rr = base + w * per_wave + g;
      const float2* pr = part_s + (static_cast<size_t>(b) * rows + (rr < rows ? rr : 0)) * nchunk_s;
      float Mr;
      double Sr;
      merge_row_stats(pr, rr < rows, nchunk_s, W, i, c, Mr, Sr);
      if (i == 0 && rr < rows) {
        sh.row_m[rr] = Mr;
        sh.row_s[rr] = Sr;
      }
    }
    __syncthreads();
    if (w == 0)
      decide_slots<kPoint>(b, c0, K, V, c, nb, nb_bad, valid, xk, uk, lt, ld, kv0, sh, out_tok,
                           out_tau, out_kv, out_p, out_q);
    __syncthreads();
  }
  const ReqState st = sh.s_st;
  if (st.m < 0) return;   // row error: nothing to draw (every workgroup of b agrees)

  const DrawRows<TIn> R = draw_rows(tgt, drf, b, K, V, st, kPoint);
  const float u_draw = uni[static_cast<size_t>(b) * (K + 1) + K];

  // ---- every draft kept (the weights are p_m of the extra row): when the statistics pass cut
  // the row into the draw's chunks, chunk j's mass is S_j 2^((M_j - M) c - log2 S) from its
  // partial, so no chunk is read for the masses and nothing is exchanged; only the workgroup of
  // the chunk holding u*Z reads its chunk, to find the token
  if (aligned && st.m == nb && !R.resid && R.mask < 0) {
    if (w == 0) {
      const float2* pr = part_s + (static_cast<size_t>(b) * rows + st.m) * nchunk_s;
      for (int j = lane; j < nchunk; j += kWave) {
        const float2 q = load_f2(pr + j);
        const double P = q.x > -INFINITY
                             ? static_cast<double>(q.y) *
                                   exp2_wide(static_cast<double>(q.x - st.M_t) *
                                                 static_cast<double>(c) -
                                             static_cast<double>(st.ls_t))
                             : 0.0;
        sh.s_cm[j] = make_double2(P, P);
      }
    }
    __syncthreads();
    if (w == 0) find_chunk(nchunk, u_draw, sh);
    __syncthreads();
    const int cs = sh.s_cs;
    if (cs < c0 || cs >= c1) return;
    const ThreadElems el = thread_elems(R.sp, V, nchunk, cv, cs, tid);
    int32_t* const out_y = out_tok + static_cast<size_t>(b) * (K + 1) + st.m;
    if constexpr (kGroups) {
      search_in_chunk<TIn, kPoint, true>(R, st, c, V, nchunk, cv, cs, el, 0.f, 0.f, sh, out_y);
    } else {
      float ws, ps;
      {
        uint4 qt[kDrawVecs], qd[kDrawVecs];
        thread_mass<kPoint>(R, st, c, V, el, qt, qd, ws, ps);
      }
      search_in_chunk<TIn, kPoint>(R, st, c, V, nchunk, cv, cs, el, ws, ps, sh, out_y);
    }
    return;
  }

  const FlaggedMasses pub{cm + static_cast<size_t>(b) * nchunk * 2};

  if constexpr (!kGroups) {
    // ---- one chunk: its masses, published; then every other chunk mass of the request into
    // LDS (the general loop below measured 0.3-0.5 us slower per C3 call in this instance).
    // The thread's vectors stay in registers for the search, the search's scan is taken while
    // the other masses arrive, and every wave finds the chunk holding u*Z itself, so the owner's
    // search runs in one wave without a workgroup barrier. That takes the draw to 5 workgroups
    // per CU, and the launch runs this instance only while its whole grid (with the key
    // selection's workgroups) fits at that occupancy.
    const int ch = c0;
    const ThreadElems el = thread_elems(R.sp, V, nchunk, cv, ch, tid);
    float ws, ps;
    uint4 qt[kDrawVecs], qd[kDrawVecs];
    thread_mass<kPoint>(R, st, c, V, el, qt, qd, ws, ps);
    double R0, P0;
    chunk_mass(ws, ps, sh.s_red, R0, P0);
    if (tid == 0) pub.publish(ch, R0, P0);
    const ScanPrep prep = scan_prep(ws, sh);
    bool missing = false;
    for (int j = tid; j < nchunk; j += kBlock) {
      double r = R0, q = P0;
      if (j != ch && !pub.poll(j, wait_polls, r, q)) {
        r = -1.0;   // marks the entry missing
        missing = true;
      }
      sh.s_cm[j] = make_double2(r, q);
    }
    if (__syncthreads_or(missing)) help_missing_masses<TIn, kPoint>(R, st, c, V, nchunk, cv, sh);
    const ChunkPick f = pick_chunk(nchunk, u_draw, sh);   // every wave: no barrier
    if (f.cs != ch) return;
    int32_t* const out_y = out_tok + static_cast<size_t>(b) * (K + 1) + st.m;
    if (!f.usep) {
      search_in_wave<TIn, kPoint>(R, st, c, V, nchunk, cv, ch, f, prep, qt, qd, sh, out_y);
      return;
    }
    // rare (round-off left no residual mass): the draw takes p, searched by the whole workgroup
    if (w == 0) find_chunk(nchunk, u_draw, sh);
    __syncthreads();
    search_in_chunk<TIn, kPoint, false, true>(R, st, c, V, nchunk, cv, ch, el, ws, ps, sh, out_y,
                                              qt, qd, &prep);
    return;
  }

  // ---- this workgroup's chunk masses, published one chunk after another (each also to LDS)
  ThreadElems el;
  float ws = 0.f, ps = 0.f;   // the thread masses of the last chunk (the only one when group = 1)
  for (int k = c0; k < c1; ++k) {
    el = thread_elems(R.sp, V, nchunk, cv, k, tid);
    {
      uint4 qt[kDrawVecs], qd[kDrawVecs];
      thread_mass<kPoint>(R, st, c, V, el, qt, qd, ws, ps);
    }
    double R0, P0;
    chunk_mass(ws, ps, sh.s_red, R0, P0);
    if (tid == 0) {
      pub.publish(k, R0, P0);
      sh.s_cm[k] = make_double2(R0, P0);
    }
  }

  // ---- gather every other chunk mass of the request into LDS; a chunk not published within the
  // poll budget is computed here (the same bits its owner publishes)
  bool missing = false;
  for (int j = tid; j < nchunk; j += kBlock) {
    if (j >= c0 && j < c1) continue;
    double r = 0.0, q = 0.0;
    if (!pub.poll(j, wait_polls, r, q)) {
      r = -1.0;   // marks the entry missing
      missing = true;
    }
    sh.s_cm[j] = make_double2(r, q);
  }
  if (__syncthreads_or(missing)) help_missing_masses<TIn, kPoint>(R, st, c, V, nchunk, cv, sh);

  if (w == 0) find_chunk(nchunk, u_draw, sh);
  __syncthreads();
  const int cs = sh.s_cs;
  if (cs < c0 || cs >= c1) return;
  int32_t* const out_y = out_tok + static_cast<size_t>(b) * (K + 1) + st.m;
  if (c1 - c0 == 1)   // uniform: the thread masses of this workgroup's one chunk are at hand
    search_in_chunk<TIn, kPoint>(R, st, c, V, nchunk, cv, cs, el, ws, ps, sh, out_y);
  else
    search_in_chunk<TIn, kPoint, true>(R, st, c, V, nchunk, cv, cs,
                                       thread_elems(R.sp, V, nchunk, cv, cs, tid), 0.f, 0.f, sh,
                                       out_y);
}


// ------------------------------------------------------------------------------ one launch
// Small batches (fused_shape_ok: every workgroup of the call resident at once) run the
// statistics and the draw in one launch. The statistics workgroups come first in the grid and
// publish their chunk (M, S) and the gathered logits as tagged words; the draw workgroups after
// them read those words instead of waiting for a kernel boundary, then publish and gather their
// chunk masses the same way. A word holds a 32-bit payload in its low half and the call's tag in
// its high half: the tag is new for every call (a host counter, never 0), so words left by
// earlier calls never match and nothing is cleared between calls. Every wait is bounded; a
// workgroup that stops waiting computes the missing item itself with the code that publishes
// it, so the bits never depend on who produced them. The merge, the slot decisions, the masses,
// the scan and the search are the two-launch draw's own functions: the outputs equal that
// path's bit for bit.

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) {
  return (static_cast<uint64_t>(tag) << 32) | v;
}
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t tag) {
  return static_cast<uint32_t>(w >> 32) == tag;
}

// A chunk's (R, P) masses as four tagged words (each float64 in two halves).
struct TaggedMasses {
  uint64_t* tm;   // [nchunk][4] of one request
  uint32_t tag;
  __device__ void publish(int j, double R, double P) const {
    const uint64_t r = dbits(R), p = dbits(P);
    store_coherent(&tm[4 * j], tagged(tag, static_cast<uint32_t>(r)));
    store_coherent(&tm[4 * j + 1], tagged(tag, static_cast<uint32_t>(r >> 32)));
    store_coherent(&tm[4 * j + 2], tagged(tag, static_cast<uint32_t>(p)));
    store_coherent(&tm[4 * j + 3], tagged(tag, static_cast<uint32_t>(p >> 32)));
  }
  // Reads chunk j's masses, re-polling at most `polls` times; false if they are not all there.
  __device__ bool poll(int j, int polls, double& R, double& P) const {
    uint64_t w0 = load_coherent(&tm[4 * j]), w1 = load_coherent(&tm[4 * j + 1]);
    uint64_t w2 = load_coherent(&tm[4 * j + 2]), w3 = load_coherent(&tm[4 * j + 3]);
    while (!(has_tag(w0, tag) && has_tag(w1, tag) && has_tag(w2, tag) && has_tag(w3, tag))) {
      if (polls-- <= 0) return false;
      __builtin_amdgcn_s_sleep(2);
      if (!has_tag(w0, tag)) w0 = load_coherent(&tm[4 * j]);
      if (!has_tag(w1, tag)) w1 = load_coherent(&tm[4 * j + 1]);
      if (!has_tag(w2, tag)) w2 = load_coherent(&tm[4 * j + 2]);
      if (!has_tag(w3, tag)) w3 = load_coherent(&tm[4 * j + 3]);
    }
    R = bits_d((w1 << 32) | static_cast<uint32_t>(w0));
    P = bits_d((w3 << 32) | static_cast<uint32_t>(w2));
    return true;
  }
};

// Chunk ch of row r of request b, as the statistics pass computes it (plain loads); (M, S) in
// thread 0. Called by the whole workgroup.
template <typename TIn>
__device__ __forceinline__ void fused_chunk_stats(const TIn* tgt, const TIn* drf, int b, int r,
                                                  int ch, int K, int V, float c, int ns, int cs,
                                                  float* sm, float* ss, float& M, float& S) {
  const TIn* row = slot_row(tgt, drf, b, r, K, V);
  const RowSpan sp = row_span(row, V);
  const ChunkRange cr = chunk_range(sp, ch, ns, cs);
  float m, s;
  thread_chunk_stats<TIn, true, false>(row, sp, cr, V, c, m, s);
  block_stats(m, s, c, sm, ss, M, S);
}

// Grid: B * (2K+1) * ns statistics workgroups (request, row, chunk), then B * nd draw
// workgroups (request, chunk of row m). part: [B][2K+1][ns][2] tagged (M, S); gath: [B][2K]
// tagged logits of the draft tokens (target slots, then draft slots); mass: [B][nd][4].
template <typename TIn>
__global__ __launch_bounds__(kBlock) void sample_fused_kernel(
    const TIn* __restrict__ tgt, const TIn* __restrict__ drf, const int32_t* __restrict__ xtok,
    const float* __restrict__ uni, const int32_t* __restrict__ kv_in, int K, int V, float c,
    int ns, int cs, int nd, int cv, int n_stats, uint32_t tag, uint64_t* __restrict__ part,
    uint64_t* __restrict__ gath, uint64_t* __restrict__ mass, int wait_polls,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_tau, int32_t* __restrict__ out_kv,
    float* __restrict__ out_p, float* __restrict__ out_q) {
  using E = Elem<TIn>;
  constexpr int N = E::N;
  __shared__ float sm[kWaves], ss[kWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int rows = 2 * K + 1;

  if (static_cast<int>(blockIdx.x) < n_stats) {
    // ---- statistics of one (request, row, chunk), as sample_stats_kernel computes them
    const int ch = blockIdx.x % ns;
    const int rb = blockIdx.x / ns;
    const int r = rb % rows, b = rb / rows;
    float M, S;
    fused_chunk_stats<TIn>(tgt, drf, b, r, ch, K, V, c, ns, cs, sm, ss, M, S);
    if (tid == 0) {
      uint64_t* pw = part + 2 * (static_cast<size_t>(rb) * ns + ch);
      store_coherent(pw, tagged(tag, __float_as_uint(M)));
      store_coherent(pw + 1, tagged(tag, __float_as_uint(S)));
      if (r != K) {   // the chunk holding the slot's draft token publishes that token's logit
        const TIn* row = slot_row(tgt, drf, b, r, K, V);
        const RowSpan sp = row_span(row, V);
        const ChunkRange cr = chunk_range(sp, ch, ns, cs);
        const int slot = r < K ? r : r - K - 1;
        const int x = xtok[static_cast<size_t>(b) * K + slot];
        const int lo = cr.first ? 0 : sp.head + cr.vbeg * N;
        const int hi = cr.last ? V : sp.head + cr.vend * N;
        if (x >= lo && x < hi)
          store_coherent(gath + static_cast<size_t>(b) * 2 * K + (r < K ? slot : K + slot),
                         tagged(tag, __float_as_uint(E::one(row, x))));
      }
    }
    return;
  }

  // ---- draw: one (request, chunk of row m)
  __shared__ DrawShared sh;
  __shared__ float2 s_part[kFusedMaxPartials];
  __shared__ float s_gath[2 * SPEC_MAX_K];
  const int dq = static_cast<int>(blockIdx.x) - n_stats;
  const int b = dq / nd, ch = dq % nd;
  const bool valid = w == 0 && lane < K;
  const int xk = valid ? xtok[static_cast<size_t>(b) * K + lane] : 0;
  const float uk = valid ? uni[static_cast<size_t>(b) * (K + 1) + lane] : 0.f;
  const int kv0 = (ch == 0 && tid == 0 && kv_in) ? kv_in[b] : 0;

  // the request's chunk partials into LDS; one not published within the poll budget is marked
  // (S = -1: a published sum is >= 0 or NaN) and computed below
  const int np = rows * ns;
  const uint64_t* pw = part + 2 * static_cast<size_t>(b) * np;
  bool miss = false;
  for (int j = tid; j < np; j += kBlock) {
    uint64_t a = load_coherent(pw + 2 * j), z = load_coherent(pw + 2 * j + 1);
    for (int polls = wait_polls; !(has_tag(a, tag) && has_tag(z, tag)) && polls > 0; --polls) {
      __builtin_amdgcn_s_sleep(2);
      if (!has_tag(a, tag)) a = load_coherent(pw + 2 * j);
      if (!has_tag(z, tag)) z = load_coherent(pw + 2 * j + 1);
    }
    const bool ok = has_tag(a, tag) && has_tag(z, tag);
    s_part[j] = ok ? make_float2(__uint_as_float(static_cast<uint32_t>(a)),
                                 __uint_as_float(static_cast<uint32_t>(z)))
                   : make_float2(0.f, -1.f);
    miss = miss || !ok;
  }
  // the draft tokens' logits; one not published in time is read here (the value its chunk
  // publishes). An out-of-range token has none: the slot decisions report it as a row error.
  for (int j = tid; j < 2 * K; j += kBlock) {
    const int slot = j < K ? j : j - K;
    const int x = xtok[static_cast<size_t>(b) * K + slot];
    float v = 0.f;
    if (x >= 0 && x < V) {
      const uint64_t* gw = gath + static_cast<size_t>(b) * 2 * K + j;
      uint64_t a = load_coherent(gw);
      for (int polls = wait_polls; !has_tag(a, tag) && polls > 0; --polls) {
        __builtin_amdgcn_s_sleep(2);
        a = load_coherent(gw);
      }
      v = has_tag(a, tag)
              ? __uint_as_float(static_cast<uint32_t>(a))
              : E::one(slot_row(tgt, drf, b, j < K ? slot : K + 1 + slot, K, V), x);
    }
    s_gath[j] = v;
  }
  if (__syncthreads_or(miss)) {
    for (int j = 0; j < np; ++j) {
      if (!(s_part[j].y < 0.f)) continue;   // uniform: read after a barrier
      float M, S;
      fused_chunk_stats<TIn>(tgt, drf, b, j / ns, j % ns, K, V, c, ns, cs, sm, ss, M, S);
      if (tid == 0) s_part[j] = make_float2(M, S);
      __syncthreads();
    }
  }

  // ---- merge and slot decisions, as the two-launch draw (partials from LDS)
  {
    const float lt = valid ? s_gath[lane] : 0.f;
    const float ld = valid ? s_gath[K + lane] : 0.f;
    const int W = merge_width(ns, rows);
    const int per_wave = kWave / W, g = lane / W, i = lane % W;
    for (int base = 0; base < rows; base += kWaves * per_wave) {
      const int rr = base + w * per_wave + g;
      const float2* pr = s_part + (rr < rows ? rr : 0) * ns;
      float Mr;
      double Sr;
      merge_row_stats_rd([pr](int j) { return pr[j]; }, rr < rows, ns, W, i, c, Mr, Sr);
      if (i == 0 && rr < rows) {
        sh.row_m[rr] = Mr;
        sh.row_s[rr] = Sr;
      }
    }
    __syncthreads();
    if (w == 0)
      decide_slots<false>(b, ch, K, V, c, K, false, valid, xk, uk, lt, ld, kv0, sh, out_tok,
                          out_tau, out_kv, out_p, out_q);
    __syncthreads();
  }
  const ReqState st = sh.s_st;
  if (st.m < 0) return;   // row error: nothing to draw (every workgroup of b agrees)

  // ---- the chunk's masses, exchanged; the chunk holding u*Z finds the token
  const DrawRows<TIn> R = draw_rows(tgt, drf, b, K, V, st, false);
  const float u_draw = uni[static_cast<size_t>(b) * (K + 1) + K];
  const TaggedMasses pub{mass + static_cast<size_t>(b) * nd * 4, tag};
  const ThreadElems el = thread_elems(R.sp, V, nd, cv, ch, tid);
  // the vectors stay in registers until the search (the grid is small: occupancy is no concern)
  float ws, ps;
  uint4 qt[kDrawVecs], qd[kDrawVecs];
  thread_mass<false>(R, st, c, V, el, qt, qd, ws, ps);
  double R0, P0;
  chunk_mass(ws, ps, sh.s_red, R0, P0);
  if (tid == 0) pub.publish(ch, R0, P0);
  const ScanPrep prep = scan_prep(ws, sh);
  bool missing = false;
  for (int j = tid; j < nd; j += kBlock) {
    double rm = R0, qm = P0;
    if (j != ch && !pub.poll(j, wait_polls, rm, qm)) {
      rm = -1.0;   // marks the entry missing
      missing = true;
    }
    sh.s_cm[j] = make_double2(rm, qm);
  }
  if (__syncthreads_or(missing)) help_missing_masses<TIn, false>(R, st, c, V, nd, cv, sh);
  {
    const ChunkPick f = pick_chunk(nd, u_draw, sh);
    if (f.cs != ch) return;
    if (!f.usep) {
      search_in_wave<TIn, false>(R, st, c, V, nd, cv, ch, f, prep, qt, qd, sh,
                                 out_tok + static_cast<size_t>(b) * (K + 1) + st.m);
      return;
    }
  }
  if (w == 0) find_chunk(nd, u_draw, sh);
  __syncthreads();
  if (sh.s_cs != ch) return;
  search_in_chunk<TIn, false, false, true>(R, st, c, V, nd, cv, ch, el, ws, ps, sh,
                                           out_tok + static_cast<size_t>(b) * (K + 1) + st.m,
                                           qt, qd, &prep);
}

// The tag of a one-launch call: a process-wide counter that skips 0 (the value of cleared
// words). A word is mistaken for a current one only if it was written exactly 2^32 calls earlier
// and has not been written since.
uint32_t next_call_tag() {
  static std::atomic<uint32_t> counter{0};
  uint32_t t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  while (t == 0) t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return t;
}

struct SamplePlan {
  KernelPlan stats, draw;
};

template <typename TIn>
SamplePlan default_sample_plan(int B, int K, int V, bool keys) {
  constexpr int N = 16 / sizeof(TIn);
  (void)keys;   // the keys path streams the rows with the same plan
  return SamplePlan{stats_plan(B, K, V, N), draw_plan(B, K, V, N)};
}

// keys: F > 0 computes outcome keys during the same two launches
struct KeyRequest {
  int F;
  int exclude;
  int32_t* out_keys;
  float* out_prob;
};

template <typename TIn, bool kKeys, bool kMixed, bool kPoint = false>
int launch_sample_t(const void* target, const void* draft, const int32_t* xtok, const float* uni,
                    const int32_t* kv_in, int B, int K, int V, float T, int32_t* out_tok,
                    int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                    size_t ws_bytes,
                    hipStream_t stream, hipEvent_t* ev, int wait_polls, const SamplePlan& P,
                    const KeyRequest& kr, const float* temps, const int32_t* dlen = nullptr) {
  const size_t g1 = static_cast<size_t>(B) * (kPoint ? K + 1 : 2 * K + 1) * P.stats.nchunk;
  const int group = draw_group(B, P.draw.nchunk);   // chunks per draw workgroup
  // the one-chunk instance, while every chunk fits on the GPU at its occupancy; otherwise the
  // grouped instance (one chunk per workgroup too, if they fit at its higher occupancy)
  const bool one_chunk = draw_one_chunk(B, P.draw.nchunk + (kKeys ? K : 0), kDrawResidentHeld);
  const size_t n_chunks = static_cast<size_t>(B) * P.draw.nchunk;
  const size_t n_draw = static_cast<size_t>(B) * ((P.draw.nchunk + group - 1) / group);
  // with keys, one more workgroup per draft slot selects that slot's keys during the draw
  const size_t g2 = n_draw + (kKeys ? static_cast<size_t>(B) * K : 0);
  if (!grid_fits(g1) || !grid_fits(g2) || P.draw.cv != kBlock * kDrawVecs ||
      P.draw.nchunk > kMaxDrawChunks)
    return SPEC_ERR_ARG;
  const WsLayout L = ws_layout(B, K, V, 1, ws_bytes);
  const float c = exp2_scale(T);
  const TIn* t = static_cast<const TIn*>(target);
  const TIn* d = static_cast<const TIn*>(draft);   // null for point-mass drafts
  float2* part1 = ws_ptr<float2>(ws, L.part_stats);
  float* gath = ws_ptr<float>(ws, L.gathered);
  uint64_t* cm = ws_ptr<uint64_t>(ws, L.part_draw);
  float* kwmax = ws_ptr<float>(ws, L.part_vwm);
  const int nclear = static_cast<int>(n_chunks * 2);
  const dim3 grid1(static_cast<unsigned>(g1)), grid2(static_cast<unsigned>(g2)), block(kBlock);
  const int ns = P.stats.nchunk, cs = P.stats.cv, nd = P.draw.nchunk, cd = P.draw.cv;
  const int polls = wait_polls < 0 ? SPEC_DEFAULT_WAIT_POLLS : wait_polls;
  const int pick = kr.F + (kr.exclude ? 1 : 0);
  const KeyArgs ka{pick, kr.F, kr.exclude, cs, kwmax, kr.out_keys, kr.out_prob};
  const int nd_wg = static_cast<int>(n_draw);
  // load hint of the statistics pass, from the bytes it streams (measured at C3 shapes cut to B
  // requests, alternating A/B: every draft row streamed at B = 32 (74 MB) and B = 64 (148 MB)
  // saved 0.5 and 0.9-1.3 us per call against ordinary loads everywhere, and streaming only the
  // later half of the slots' draft rows saved another 0.3 and 0.7-0.8 us; at B <= 16 (37 MB and
  // less) the call is latency-bound and nothing changed, at B = 1 it lost 0.4 us; a mixed batch
  // lost 1 us)
  const long long streamed =
      static_cast<long long>(B) * (kPoint ? K + 1 : 2 * K + 1) * V *
      static_cast<long long>(sizeof(TIn));
  const int nt = streamed > kInfinityCacheBytes ? kHintStream
                 : (!kMixed && !kPoint && streamed >= kInfinityCacheBytes / 4)
                     ? kHintStreamDraft
                     : kHintCached;
  // the statistics pass cut every row into the draw's chunks (chunk masses of an extra row can be
  // taken from its partials)
  const int aligned = (ns == nd && cs == cd) ? 1 : 0;
  if constexpr (!kKeys && !kMixed && !kPoint) {
    // small batches: one launch, unless the call is timed by events or captured into a graph (a
    // replay would repeat the tag, and words of the previous replay would match it)
    constexpr int kEpv = 16 / static_cast<int>(sizeof(TIn));
    hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
    if (ev == nullptr && fused_shape_ok(B, K, V, kEpv) &&
        hipStreamIsCapturing(stream, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
      const FusedWords fw = fused_words(B, K, V, kEpv);
      unsigned char* base = static_cast<unsigned char*>(ws) + L.fused;
      const int n_stats = static_cast<int>(g1);
      hipLaunchKernelGGL((sample_fused_kernel<TIn>), dim3(static_cast<unsigned>(g1 + n_draw)),
                         block, 0, stream, t, d, xtok, uni, kv_in, K, V, c, ns, cs, nd, cd,
                         n_stats, next_call_tag(), reinterpret_cast<uint64_t*>(base + fw.part),
                         reinterpret_cast<uint64_t*>(base + fw.gath),
                         reinterpret_cast<uint64_t*>(base + fw.mass), polls, out_tok, out_tau,
                         out_kv, out_p, out_q);
      return launch_status();
    }
  }
  if (ev == nullptr) {
    hipLaunchKernelGGL((sample_stats_kernel<TIn, kKeys, kMixed, kPoint>), grid1, block, 0, stream,
                       t, d, xtok, K, V, c, ns, cs, part1, gath, cm, nclear, kwmax, temps, dlen,
                       nt);
    if (!one_chunk)
      hipLaunchKernelGGL((sample_draw_kernel<TIn, kKeys, kMixed, kPoint, true>), grid2, block, 0,
                         stream, t, d, xtok, uni, kv_in, K, V, c, ns,
                         static_cast<const float2*>(part1), static_cast<const float*>(gath), nd,
                         cd, aligned, group, cm, polls, out_tok, out_tau, out_kv, out_p, out_q, ka,
                         temps, dlen, nd_wg);
    else
      hipLaunchKernelGGL((sample_draw_kernel<TIn, kKeys, kMixed, kPoint, false>), grid2, block, 0,
                         stream, t, d, xtok, uni, kv_in, K, V, c, ns,
                         static_cast<const float2*>(part1), static_cast<const float*>(gath), nd,
                         cd, aligned, 1, cm, polls, out_tok, out_tau, out_kv, out_p, out_q, ka,
                         temps, dlen, nd_wg);
  } else {
    // profiling: the runtime records the events at each kernel's start and end
    hipExtLaunchKernelGGL((sample_stats_kernel<TIn, kKeys, kMixed, kPoint>), grid1, block, 0,
                          stream, ev[0], ev[1], 0, t, d, xtok, K, V, c, ns, cs, part1, gath, cm,
                          nclear, kwmax, temps, dlen, nt);
    if (!one_chunk)
      hipExtLaunchKernelGGL((sample_draw_kernel<TIn, kKeys, kMixed, kPoint, true>), grid2, block,
                            0, stream, ev[2], ev[3], 0, t, d, xtok, uni, kv_in, K, V, c, ns,
                            static_cast<const float2*>(part1), static_cast<const float*>(gath),
                            nd, cd, aligned, group, cm, polls, out_tok, out_tau, out_kv, out_p,
                            out_q, ka, temps, dlen, nd_wg);
    else
      hipExtLaunchKernelGGL((sample_draw_kernel<TIn, kKeys, kMixed, kPoint, false>), grid2, block,
                            0, stream, ev[2], ev[3], 0, t, d, xtok, uni, kv_in, K, V, c, ns,
                            static_cast<const float2*>(part1), static_cast<const float*>(gath),
                            nd, cd, aligned, 1, cm, polls, out_tok, out_tau, out_kv, out_p, out_q,
                            ka, temps, dlen, nd_wg);
  }
  return launch_status();
}

template <typename TIn>
int launch_sample(const void* target, const void* draft, const int32_t* xtok, const float* uni,
                  const int32_t* kv_in, int B, int K, int V, float T, int32_t* out_tok,
                  int32_t* out_tau, int32_t* out_kv, float* out_p, float* out_q, void* ws,
                  size_t ws_bytes, hipStream_t stream, hipEvent_t* ev, int wait_polls,
                  const KeyRequest& kr,
                  const float* temps) {
  const bool keys = kr.F > 0;
  const SamplePlan P = default_sample_plan<TIn>(B, K, V, keys);
  if (temps != nullptr)
    return launch_sample_t<TIn, false, true>(target, draft, xtok, uni, kv_in, B, K, V, T, out_tok,
                                             out_tau, out_kv, out_p, out_q, ws, ws_bytes, stream,
                                             ev, wait_polls, P, kr, temps);
  if (keys)
    return launch_sample_t<TIn, true, false>(target, draft, xtok, uni, kv_in, B, K, V, T, out_tok,
                                             out_tau, out_kv, out_p, out_q, ws, ws_bytes, stream,
                                             ev, wait_polls, P, kr, nullptr);
  return launch_sample_t<TIn, false, false>(target, draft, xtok, uni, kv_in, B, K, V, T, out_tok,
                                            out_tau, out_kv, out_p, out_q, ws, ws_bytes, stream,
                                            ev, wait_polls, P, kr, nullptr);
}

// Host-side checks of a sampling call's arguments other than its workspace, in the order the
// header documents.
int check_sample_args(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                      float temperature, const int32_t* out_tokens, const int32_t* out_tau,
                      const KeyRequest& kr, const float* temps) {
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (check_logits(target_logits, dtype) != SPEC_OK ||
      check_logits(draft_logits, dtype) != SPEC_OK || draft_tokens == nullptr ||
      uniforms == nullptr || out_tokens == nullptr || out_tau == nullptr)
    return SPEC_ERR_ARG;
  if (kr.F != 0) {
    const int pick = kr.F + (kr.exclude ? 1 : 0);
    if (kr.F < 1 || pick > SPEC_MAX_F || pick > V || kr.out_keys == nullptr) return SPEC_ERR_ARG;
  }
  if (temps == nullptr && (!std::isfinite(temperature) || !(temperature > 0.f) ||
                           !std::isfinite(exp2_scale(temperature))))
    return SPEC_ERR_TEMPERATURE;
  return SPEC_OK;
}

int verify_sample_entry(const void* target_logits, const void* draft_logits, int dtype,
                        const int32_t* draft_tokens, const float* uniforms,
                        const int32_t* kv_len_in, int B, int K, int V, float temperature,
                        int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                        float* out_q, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t* events, int wait_polls,
                        const KeyRequest& kr, const float* temps = nullptr) {
  int rc = check_sample_args(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K,
                             V, temperature, out_tokens, out_tau, kr, temps);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, 1)) != SPEC_OK) return rc;
  if (events != nullptr)
    for (int i = 0; i < 4; ++i)
      if (events[i] == nullptr) return SPEC_ERR_ARG;
  if (dtype == SPEC_BF16)
    return launch_sample<uint16_t>(target_logits, draft_logits, draft_tokens, uniforms, kv_len_in,
                                   B, K, V, temperature, out_tokens, out_tau, out_kv_len, out_p,
                                   out_q, workspace, workspace_bytes, stream, events, wait_polls,
                                   kr, temps);
  return launch_sample<float>(target_logits, draft_logits, draft_tokens, uniforms, kv_len_in, B,
                              K, V, temperature, out_tokens, out_tau, out_kv_len, out_p, out_q,
                              workspace, workspace_bytes, stream, events, wait_polls, kr, temps);
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
                                 nullptr, -1, sv::KeyRequest{0, 0, nullptr, nullptr});
}

// ------------------------------------------------------------------------------ no allocation
// The workspace of spec_verify_sample_noalloc, for callers that cannot allocate one: one array
// per GPU, loaded with the code object and held until the process ends. In host code this name
// is a host-side stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, once per device (scratch_address below), and only that address is ever
// passed to a kernel. Nothing in it has to start at zero: in the two-launch form the streaming
// kernel clears the published-mass words its draw polls, in the one-launch form every polled word
// carries the call's tag, and every other region is written before it is read.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace sv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on its first use there).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SPEC_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace
}  // namespace sv

extern "C" int spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits,
                                          int dtype, const int32_t* draft_tokens,
                                          const float* uniforms, const int32_t* kv_len_in, int B,
                                          int K, int V, float temperature, int32_t* out_tokens,
                                          int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                                          float* out_q, hipStream_t stream) {
  using namespace sv;
  // every host-side check first, so a call that cannot run touches no device
  const KeyRequest none{0, 0, nullptr, nullptr};
  int rc = check_sample_args(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V,
                             temperature, out_tokens, out_tau, none, nullptr);
  if (rc != SPEC_OK) return rc;
  if (ws_layout(B, K, V, 1, 0).total > static_cast<size_t>(SPEC_NOALLOC_SCRATCH_BYTES))
    return SPEC_ERR_SCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != SPEC_OK) return rc;
  return verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                             kv_len_in, B, K, V, temperature, out_tokens, out_tau, out_kv_len,
                             out_p, out_q, ws, SPEC_NOALLOC_SCRATCH_BYTES, stream, nullptr, -1,
                             none);
}

extern "C" int spec_verify_sample_ex(const void* target_logits, const void* draft_logits,
                                     int dtype, const int32_t* draft_tokens,
                                     const float* uniforms, const int32_t* kv_len_in, int B,
                                     int K, int V, float temperature, int32_t* out_tokens,
                                     int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                                     float* out_q, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, hipEvent_t* events, int wait_polls) {
  return sv::verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                 kv_len_in, B, K, V, temperature, out_tokens, out_tau,
                                 out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
                                 events, wait_polls, sv::KeyRequest{0, 0, nullptr, nullptr});
}

extern "C" int spec_verify_sample_keys(const void* target_logits, const void* draft_logits,
                                       int dtype, const int32_t* draft_tokens,
                                       const float* uniforms, const int32_t* kv_len_in, int B,
                                       int K, int V, float temperature, int F, int exclude_draft,
                                       int32_t* out_tokens, int32_t* out_tau,
                                       int32_t* out_kv_len, float* out_p, float* out_q,
                                       int32_t* out_keys, float* out_key_prob, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (F < 1) return SPEC_ERR_ARG;
  return sv::verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                 kv_len_in, B, K, V, temperature, out_tokens, out_tau,
                                 out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
                                 nullptr, -1,
                                 sv::KeyRequest{F, exclude_draft ? 1 : 0, out_keys, out_key_prob});
}

extern "C" int spec_verify_mixed(const void* target_logits, const void* draft_logits, int dtype,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const int32_t* kv_len_in, const float* temperatures, int B,
                                 int K, int V, int32_t* out_tokens, int32_t* out_tau,
                                 int32_t* out_kv_len, float* out_p, float* out_q,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (temperatures == nullptr) return SPEC_ERR_ARG;
  return sv::verify_sample_entry(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                 kv_len_in, B, K, V, 1.f, out_tokens, out_tau, out_kv_len, out_p,
                                 out_q, workspace, workspace_bytes, stream, nullptr, -1,
                                 sv::KeyRequest{0, 0, nullptr, nullptr}, temperatures);
}

extern "C" int spec_verify_point(const void* target_logits, int dtype,
                                 const int32_t* draft_tokens, const int32_t* draft_len,
                                 const float* uniforms, const int32_t* kv_len_in, int B, int K,
                                 int V, float temperature, int32_t* out_tokens, int32_t* out_tau,
                                 int32_t* out_kv_len, float* out_p, float* out_q,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace sv;
  int rc = check_dtype(dtype);
  if (rc != SPEC_OK) return rc;
  if ((rc = check_dims(B, K, V)) != SPEC_OK) return rc;
  if (check_logits(target_logits, dtype) != SPEC_OK || draft_tokens == nullptr ||
      out_tokens == nullptr || out_tau == nullptr)
    return SPEC_ERR_ARG;
  if (!(temperature == 0.f) &&
      (!std::isfinite(temperature) || !(temperature > 0.f) ||
       !std::isfinite(exp2_scale(temperature))))
    return SPEC_ERR_TEMPERATURE;
  if ((rc = check_workspace(workspace, workspace_bytes, B, K, V, 1)) != SPEC_OK) return rc;
  if (temperature == 0.f)
    return greedy_point_entry(target_logits, dtype, draft_tokens, draft_len, kv_len_in, B, K, V,
                              out_tokens, out_tau, out_kv_len, out_p, out_q, workspace,
                              workspace_bytes, stream);
  if (uniforms == nullptr) return SPEC_ERR_ARG;
  const KeyRequest none{0, 0, nullptr, nullptr};
  if (dtype == SPEC_BF16)
    return launch_sample_t<uint16_t, false, false, true>(
        target_logits, nullptr, draft_tokens, uniforms, kv_len_in, B, K, V, temperature,
        out_tokens, out_tau, out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
        nullptr, -1, SamplePlan{point_plan(B, K, V, 8), draw_plan(B, K, V, 8)}, none, nullptr,
        draft_len);
  return launch_sample_t<float, false, false, true>(
      target_logits, nullptr, draft_tokens, uniforms, kv_len_in, B, K, V, temperature,
      out_tokens, out_tau, out_kv_len, out_p, out_q, workspace, workspace_bytes, stream,
      nullptr, -1, SamplePlan{point_plan(B, K, V, 4), draw_plan(B, K, V, 4)}, none, nullptr,
      draft_len);
}
