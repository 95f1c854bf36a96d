// Chunk plans and workspace layout, shared by the host launchers and the kernels.
//
// A logit row of V elements is cut into chunks of `cv` 16-byte vectors; each chunk is one
// workgroup's work item. The plan depends only on the sizes and the element size, so every row
// of a launch has the same number of chunks (a row's own head/tail split can move its vector
// count down by one, which only shortens its last chunk).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef __HIPCC__
#define SV_HD
#else
#define SV_HD __host__ __device__
#endif

namespace sv {

constexpr int kBlock = 256;            // threads per workgroup, every kernel
constexpr int kVecPerThread = 4;       // 16-byte vectors a thread holds per pass
constexpr int kPassVecs = kBlock * kVecPerThread;
constexpr int kCUs = 256;              // MI355X compute units

// Streaming plan of one kernel: every row is cut into `nchunk` chunks of `cv` vectors (the last
// one shorter); one workgroup per (row, chunk).
struct KernelPlan {
  int cv;
  int nchunk;
};

SV_HD inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Chunking for `rows` rows of V elements, `epv` elements per 16-byte vector, for a kernel of
// which `resident` workgroups fit on one CU at a time. Small chunks (one pass of the block,
// 16 KiB of bf16) balance best when they make many rounds of workgroups; when they would not,
// the rows are cut into as many equal chunks as fill the GPU once (down to one vector per
// thread), so no partial second round of workgroups is left running alone and small batches
// still spread over all CUs. `max_cv` caps the chunk (0 = no cap).
SV_HD inline KernelPlan plan_rows(int rows, int V, int epv, int resident, int max_cv = 0) {
  const int nvec = V / epv > 0 ? V / epv : 1;
  const int cap = kCUs * resident;
  int nchunk = ceil_div(nvec, kPassVecs);
  if (static_cast<long long>(rows) * nchunk < 4ll * cap) {
    const int fill = cap / rows;
    const int finest = ceil_div(nvec, kBlock);   // one vector per thread
    nchunk = fill < 1 ? 1 : (fill < finest ? fill : finest);
  }
  int cv = ceil_div(ceil_div(nvec, nchunk), kBlock) * kBlock;   // balanced, whole 256-vector steps
  if (max_cv > 0 && cv > max_cv) cv = max_cv;
  return KernelPlan{cv, ceil_div(nvec, cv)};
}

// MI355X's Infinity Cache (the memory-side cache in front of HBM), bytes
constexpr long long kInfinityCacheBytes = 256ll << 20;

// workgroups per CU at once, from the compiler's resource report for gfx950
constexpr int kStatsResident = 8;
constexpr int kGreedyResident = 8;
constexpr int kPredictResident = 8;

SV_HD inline KernelPlan stats_plan(int B, int K, int V, int epv) {
  return plan_rows(B * (2 * K + 1), V, epv, kStatsResident);
}
// the draw re-reads one row (two when m < K) per request, kDrawVecs adjacent vectors per thread,
// and keeps them in registers for the final search
constexpr int kDrawVecs = 4;
SV_HD inline KernelPlan draw_plan(int B, int K, int V, int epv) {
  (void)B;
  (void)K;
  const int nvec = V / epv > 0 ? V / epv : 1;
  return KernelPlan{kBlock * kDrawVecs, ceil_div(nvec, kBlock * kDrawVecs)};
}
// Draw workgroups per CU at once (from the compiler's resource report for gfx950: registers and
// LDS both allow eight), and five for the one-chunk instance that holds each thread's vectors
// across the mass exchange (92-93 registers; 84-86 for fp32 rows).
constexpr int kDrawResident = 8;
constexpr int kDrawResidentHeld = 5;
// Consecutive chunks of row m that one draw workgroup takes: one while every request's chunks fit
// on the GPU at once; otherwise as many as bring the draw's workgroups down to one round (at most
// kMaxDrawGroup). A workgroup whose chunks are all resident never waits for a workgroup that has
// not started, and each extra round would cost the whole chain of a draw workgroup again.
constexpr int kMaxDrawGroup = 4;
SV_HD inline int draw_group(int B, int nchunk) {
  const long long chunks = static_cast<long long>(B) * nchunk;
  const long long slots = static_cast<long long>(kCUs) * kDrawResident;
  const long long g = (chunks + slots - 1) / slots;
  return g < 1 ? 1 : (g > kMaxDrawGroup ? kMaxDrawGroup : static_cast<int>(g));
}
// Small batches run the statistics and the draw of a sampling call in one launch when every
// workgroup of it can be resident at once and the draw's merge can hold a request's chunk
// partials in LDS; the statistics chunks must not be the draw's chunks (the all-kept shortcut
// of the two-launch draw reads the partials of exactly those chunks).
constexpr int kFusedMaxPartials = 1024;   // chunk partials of one request, held in LDS
constexpr int kFusedMaxGrid = 1024;       // workgroups of one launch
SV_HD inline bool fused_shape_ok(int B, int K, int V, int epv) {
  const KernelPlan s = stats_plan(B, K, V, epv), d = draw_plan(B, K, V, epv);
  const long long rows = 2ll * K + 1;
  const long long grid = static_cast<long long>(B) * (rows * s.nchunk + d.nchunk);
  const bool aligned = s.nchunk == d.nchunk && s.cv == d.cv;
  return !aligned && rows * s.nchunk <= kFusedMaxPartials && grid <= kFusedMaxGrid &&
         draw_group(B, d.nchunk) == 1;
}
// Whether the draw runs its one-chunk instance: `per_request` workgroups per request (one per
// chunk, plus one per slot with outcome keys), every one of them resident at once at `resident`
// workgroups per CU.
SV_HD inline bool draw_one_chunk(int B, int per_request, int resident) {
  return static_cast<long long>(B) * per_request <= static_cast<long long>(kCUs) * resident;
}
// point-mass drafts: the statistics pass streams only the K+1 target rows, in chunks of at most
// one pass of the block (16 KiB of bf16) so that even a batch that would fill the GPU once with
// larger chunks runs in several rounds (measured faster: the pass has no per-workgroup handshake)
SV_HD inline KernelPlan point_plan(int B, int K, int V, int epv) {
  return plan_rows(B * (K + 1), V, epv, kStatsResident, kPassVecs);
}
// greedy verification: chunks of at most one pass of the block, so that even a batch that would
// fill the GPU once with larger chunks runs in several rounds (no workgroup waits on another)
SV_HD inline KernelPlan greedy_plan(int B, int K, int V, int epv) {
  return plan_rows(B * (K + 1), V, epv, kGreedyResident, kPassVecs);
}
// outcome keys: chunks of at most kPredictVecs vectors, so that even a batch that would fill the
// GPU once with larger chunks runs in several rounds and the workgroups' arithmetic overlaps the
// loads of others
constexpr int kPredictVecs = 1024;
SV_HD inline KernelPlan predict_plan(int B, int K, int V, int epv) {
  return plan_rows(B * K, V, epv, kPredictResident, kPredictVecs);
}

// per-request outcome of the slot scan, as the draw needs it
struct ReqState {
  int m;          // first rejected slot (K when all kept), -1 for a row error
  int xm;         // point-mass drafts: the rejected draft token, removed from the residual (-1)
  float M_t;      // maximum of the target row the draw reads (p = 2^((l - M_t) c - ls_t))
  float ls_t;     // log2 S_t of that row
  float M_d;      // same for the draft row of slot m (unused when m == K)
  float ls_d;
};

struct WsLayout {
  size_t greedy_mark;   // unsigned at offset 0 for every shape: set once a greedy decider
                        // stopped waiting (cleared only by spec_workspace_init)
  size_t greedy_words;  // 8 B [B*(K+1)*nchunk]: greedy, published chunk (max, lowest index)
  size_t words_end;     // end of the first half's regions
  size_t gathered;   // float [B*2K]: target and draft logit of each slot's draft token
  size_t part_stats; // 8 B [B*(2K+1)*nchunk] (point drafts: [B*(K+1)*nchunk]): chunk (max, sum)
  size_t part_draw;  // 16 B [B*nchunk]: published chunk (residual mass, target mass)
  size_t part_pred;  // 8 B [B*K*nchunk]: outcome keys, chunk (max, scaled sum)
  size_t part_pwm;   // 4 B [B*K*nchunk*4]: outcome keys, wave maxima
  size_t part_vwm;   // 4 B [B*K*nchunk*4]: wave maxima of the draft rows (outcome keys)
  size_t fused;      // one-launch sampling (small batches only): tagged words, FusedWords below
  size_t data_end;   // end of the last data region
  size_t total;      // bytes this shape needs: twice the larger of the two halves' regions
  bool fits;         // the caller's workspace holds this shape's words and data
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Tagged 64-bit words of the one-launch sampling path, relative to WsLayout::fused: chunk
// partials [B][2K+1][nchunk_s][2] (max, sum), gathered logits [B][2K], chunk masses
// [B][nchunk_d][4] (residual and target mass, each in two halves).
struct FusedWords {
  size_t part, gath, mass, bytes;
};
inline FusedWords fused_words(int B, int K, int V, int epv) {
  FusedWords f{0, 0, 0, 0};
  if (!fused_shape_ok(B, K, V, epv)) return f;
  const size_t b = static_cast<size_t>(B), rows = 2 * static_cast<size_t>(K) + 1;
  const size_t ns = static_cast<size_t>(stats_plan(B, K, V, epv).nchunk);
  const size_t nd = static_cast<size_t>(draw_plan(B, K, V, epv).nchunk);
  f.gath = align256(16 * b * rows * ns);
  f.mass = f.gath + align256(8 * b * 2 * static_cast<size_t>(K));
  f.bytes = f.mass + align256(32 * b * nd);
  return f;
}

template <typename PlanFn>
inline size_t max_chunks(PlanFn fn, int B, int K, int V) {
  const int a = fn(B, K, V, 4).nchunk, b = fn(B, K, V, 8).nchunk;
  return static_cast<size_t>(a > b ? a : b);
}

// Layout covering both element types. The workspace is cut in two halves. The first holds the
// greedy path's published words, zero between calls (each decider clears the words it read), and
// the greedy mark at offset 0 whatever the shape, so that calls of every shape see it. The
// second holds every other region, which each call writes before it reads. One workspace can
// therefore serve calls of different shapes in turn. `ws_bytes` is the caller's workspace size;
// `total`, the size this shape needs, does not depend on it.
inline WsLayout ws_layout(int B, int K, int V, int F, size_t ws_bytes) {
  (void)F;   // the keys go to the caller's outputs
  const size_t b = static_cast<size_t>(B), k = static_cast<size_t>(K);
  const size_t ns = max_chunks(stats_plan, B, K, V);
  const size_t npt = max_chunks(point_plan, B, K, V);
  const size_t nd = max_chunks(draw_plan, B, K, V);
  const size_t ng = max_chunks(greedy_plan, B, K, V);
  const size_t np = max_chunks(predict_plan, B, K, V);
  WsLayout L;
  L.greedy_mark = 0;
  L.greedy_words = 256;
  L.words_end = align256(L.greedy_words + 8 * b * (k + 1) * ng);
  // data regions, first relative to the start of the second half
  size_t d = 0;
  L.gathered = d;
  d = align256(d + sizeof(float) * 2 * b * k);
  L.part_stats = d;
  d = align256(d + 8 * (b * (2 * k + 1) * ns > b * (k + 1) * npt ? b * (2 * k + 1) * ns
                                                                  : b * (k + 1) * npt));
  L.part_draw = d;
  d = align256(d + 16 * b * nd);
  L.part_pred = d;
  d = align256(d + 8 * b * k * np);
  L.part_pwm = d;
  d = align256(d + 4 * b * k * np * 4);
  L.part_vwm = d;
  d = align256(d + 4 * b * k * ns * 4);
  L.fused = d;
  {
    const size_t f4 = fused_words(B, K, V, 4).bytes, f8 = fused_words(B, K, V, 8).bytes;
    d += f4 > f8 ? f4 : f8;
  }
  const size_t need_half = L.words_end > d ? L.words_end : d;
  L.total = 2 * need_half;
  const size_t half = (ws_bytes / 2) & ~static_cast<size_t>(255);
  L.fits = L.words_end <= half && half + d <= ws_bytes;
  L.gathered += half;
  L.part_stats += half;
  L.part_draw += half;
  L.part_pred += half;
  L.part_pwm += half;
  L.part_vwm += half;
  L.fused += half;
  L.data_end = half + d;
  return L;
}

}  // namespace sv
