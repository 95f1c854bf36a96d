/*
 * spec_verify.h — C ABI of libspecverify.so: the target-side verification step of speculative
 * decoding (speculative sampling) on an MI355X (gfx950) GPU.
 *
 * Sources (page titles and sections):
 *   [SD]  "speculative decodingとは" (lotook.com), section "speculative decodingはどのような手順で
 *         動くのか?": stage 2 (one target pass gives a distribution for every draft slot plus one
 *         more), stage 3 (left-to-right accept/reject; argmax match at temperature zero, a token
 *         the target likes at least as much always kept, otherwise kept by the probability
 *         ratio), stage 4 (at the first mismatch m, resample from the residual of both models'
 *         probabilities; if all K drafts are kept, draw a bonus token from the extra row);
 *         section "speculative decodingとKV cache、プロンプトキャッシュの関係は?" (both KV caches
 *         are rewound past the rejected entries).
 *   [SSD] "Speculative Speculative Decoding (SSD)" (jiwasawa.github.io), section
 *         "1. Outcome Prediction (The Saguaro Cache)": a verification outcome is (how many drafts
 *         were kept, which token the target placed); the placed token is predicted from the
 *         draft's top logits.
 *   [D3D] "LLMの生成を5倍速くする「D3D」を図で読む" (animemo.app), sections "検証のしくみ①"
 *         (row k of the target belongs to draft slot k; the row after the last draft is the
 *         bonus row), "検証のしくみ③" and "検証のまとめ" (keep, discard from the first miss,
 *         place the target's own token; tau = tokens advanced), "答え:…" (an outcome is the kept
 *         count and the placed token).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device, row-major, contiguous:
 *       target_logits [B, K+1, V]  row k is the target's distribution for draft slot k,
 *                                  row K the extra (bonus) row;
 *       draft_logits  [B, K,   V]  row k is the draft's distribution for slot k;
 *       draft_tokens  [B, K] int32; uniforms [B, K+1] float32 in [0,1): uniforms[b][k] (k<K)
 *       decides slot k, uniforms[b][K] drives the residual or bonus draw.
 *     Logit element type is SPEC_F32 (float) or SPEC_BF16 (bfloat16 bit patterns, 2 bytes);
 *     logit pointers must be aligned to their element size. 2 <= V <= SPEC_MAX_V.
 *   - -inf logits are masked tokens (probability 0). NaN or +inf logits, or a row whose logits
 *     are all -inf, give undefined (but in-bounds, terminating) results.
 *   - The caller owns every buffer, including the workspace. The library allocates nothing and
 *     keeps no mutable global state (the one exception is spec_verify_sample_noalloc's fixed
 *     per-GPU scratch array, below); calls only enqueue work on `stream` and return. Outputs
 *     are valid after the stream is synchronised. Every element of every non-null output is
 *     written.
 *   - Workspace: size from spec_workspace_bytes(B,K,V,F) (one size serves every entry point),
 *     256-byte aligned, zeroed once by spec_workspace_init before its first use. Each call
 *     leaves it ready for the next one: the greedy path's published words are cleared on the
 *     device by the workgroups that read them, and the sampling draw's published-mass words
 *     are cleared by the same call's streaming pass before the draw reads them. The greedy
 *     words live in the workspace's first half and every other region in its second, so one
 *     workspace serves calls of any shapes for which it holds at least spec_workspace_bytes
 *     (a workspace sized for the largest B, K, V a caller uses does; a call for which it is
 *     smaller returns SPEC_ERR_WORKSPACE). One workspace must not be used by two calls that
 *     may run concurrently (two streams, or two host threads on one stream without ordering):
 *     they would race.
 *   - Errors found on the host are returned synchronously, before anything is enqueued:
 *       SPEC_ERR_ARG         null required pointer, B < 1, K < 1 or K > SPEC_MAX_K, V < 2
 *                            or V > SPEC_MAX_V,
 *                            F outside [1, min(V, SPEC_MAX_F)], misaligned logit pointer,
 *                            or a launch grid that would exceed 2^31-1 blocks;
 *       SPEC_ERR_DTYPE       dtype not SPEC_F32 / SPEC_BF16;
 *       SPEC_ERR_TEMPERATURE sampling with T not finite or T <= 0 (or log2(e)/T not finite);
 *                            greedy with T != 0; prediction with T < 0 or not finite;
 *       SPEC_ERR_WORKSPACE   workspace null, not 256-byte aligned, or smaller than
 *                            spec_workspace_bytes for this call's sizes;
 *       SPEC_ERR_HIP         a launch failed (hipGetLastError after enqueueing).
 *   - Errors in device data are reported per request ("row error"): a draft token outside
 *     [0,V), or, when sampling, a draft token whose draft logit is -inf (it cannot be a sample
 *     of the draft), make that request write tau = -1, tokens all -1, kv_out = kv_in, and NaN
 *     probabilities.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 9
#define SPEC_MAX_K 64
#define SPEC_MAX_NGRAM 64
#define SPEC_MAX_CONTEXT 1073741824 /* 2^30 tokens per context row */
#define SPEC_MAX_F 16
#define SPEC_MAX_V 4194304 /* 2^22 */
#define SPEC_DEFAULT_WAIT_POLLS 16384
#define SPEC_NOALLOC_SCRATCH_BYTES 16777216 /* 16 MiB per GPU, spec_verify_sample_noalloc */

/* logit element types */
#define SPEC_F32 0
#define SPEC_BF16 1

/* status codes */
#define SPEC_OK 0
#define SPEC_ERR_ARG (-1)
#define SPEC_ERR_DTYPE (-2)
#define SPEC_ERR_TEMPERATURE (-3)
#define SPEC_ERR_WORKSPACE (-4)
#define SPEC_ERR_HIP (-5)
#define SPEC_ERR_SCRATCH (-6)

/* Returns SPEC_ABI_VERSION of the built library. */
int spec_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* spec_status_string(int status);

/* Workspace bytes needed by any entry point for these sizes (F is the largest fan-out that
 * will be passed to spec_predict_outcomes; pass 1 if prediction is not used). Returns 0 when
 * the sizes are invalid (same rules as SPEC_ERR_ARG). */
size_t spec_workspace_bytes(int B, int K, int V, int F);

/* Zeroes the workspace on `stream` (one small fill kernel): the greedy path's published words
 * and its mark. Call once after allocating a workspace. Every call leaves the workspace ready
 * for the next; only the greedy path's last-resort mark (spec_verify_greedy_ex) needs this call
 * again to be cleared. */
int spec_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Speculative-sampling verification at temperature T > 0 ([SD] stages 3-4; [D3D] 検証のまとめ).
 *   p_k = softmax(target_logits[b,k,:] / T), q_k = softmax(draft_logits[b,k,:] / T).
 *   Slots k = 0..K-1 in order: kept iff uniforms[b,k] < r_k, r_k = 1 if p_k(x_k) >= q_k(x_k),
 *   else p_k(x_k)/q_k(x_k). m = first slot not kept (K if all kept).
 *   Draw y with u = uniforms[b,K] by inverse CDF (smallest v whose running sum in token order
 *   exceeds u * total) from w = max(0, p_m - q_m) if m < K, or w = p_K if m = K.
 * Outputs (device):
 *   out_tokens [B,K+1] int32   x_0..x_{m-1}, y, then -1 padding
 *   out_tau    [B]     int32   m + 1 (tokens advanced this round)
 *   out_kv_len [B]     int32   kv_len_in[b] + tau (nullable; kv_len_in may be NULL = 0)
 *   out_p, out_q [B,K] float   p_k(x_k), q_k(x_k) for every slot (nullable)
 * Inputs are read once in one streaming pass; the target and draft rows of slot m are read
 * again by the draw (only the extra target row when every draft is kept). The pass and the draw
 * are two kernels on `stream`; for small batches (every workgroup of both fitting on the GPU at
 * once, e.g. one request at V = 32000) they are one kernel whose workgroups hand results over
 * through tagged workspace words, except while `stream` is being captured into a HIP graph
 * (a replay would repeat the call's tag), where the two kernels are recorded. Both give the same
 * outputs bit for bit. */
int spec_verify_sample(const void* target_logits, const void* draft_logits, int dtype,
                       const int32_t* draft_tokens, const float* uniforms,
                       const int32_t* kv_len_in, int B, int K, int V, float temperature,
                       int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len,
                       float* out_p, float* out_q,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* spec_verify_sample with two extra controls, for profiling and testing. Results are identical
 * to spec_verify_sample, bit for bit, whatever the controls are.
 *   events     NULL, or four caller-created hipEvent_t (timing enabled, none NULL, else
 *              SPEC_ERR_ARG): the runtime records events[0]/events[1] at the start/end of the
 *              streaming statistics kernel and events[2]/events[3] at the start/end of the draw
 *              kernel (hipExtLaunchKernelGGL). With events a small batch runs as two kernels
 *              too, so that each can be timed.
 *   wait_polls the draw's workgroups of one request exchange their chunk masses (and, in
 *              the one-kernel form, read the pass's chunk statistics and draft-token logits
 *              from the workgroups that publish them); a workgroup re-polls for such a value at
 *              most this many times (a short sleep apart) before computing it itself. Negative
 *              selects SPEC_DEFAULT_WAIT_POLLS (what spec_verify_sample uses); 0 makes every
 *              workgroup compute each value it does not find already published, which
 *              exercises that path. */
int spec_verify_sample_ex(const void* target_logits, const void* draft_logits, int dtype,
                          const int32_t* draft_tokens, const float* uniforms,
                          const int32_t* kv_len_in, int B, int K, int V, float temperature,
                          int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len,
                          float* out_p, float* out_q,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          hipEvent_t* events, int wait_polls);

/* spec_verify_sample without a workspace argument, for callers that cannot allocate one: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine): its workspace is a
 * fixed array of SPEC_NOALLOC_SCRATCH_BYTES (16 MiB) in device memory, one per GPU, loaded with
 * the library's code and held until the process ends; its device address is looked up once
 * per device on the first call there. Every other argument, every output and every result are
 * those of spec_verify_sample, bit for bit (the same kernels).
 *   Limit: sizes for which spec_workspace_bytes(B, K, V, 1) exceeds SPEC_NOALLOC_SCRATCH_BYTES
 *   (e.g. B = 64, K = 4, V = 128256 needs 1 MiB; B = 256, K = 8, V = 152064 needs 8.8 MiB) are
 *   rejected with SPEC_ERR_SCRATCH before anything touches the device.
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (nothing in it needs clearing: each call clears what its draw polls). Calls that
 *   may overlap on one GPU (two streams, or two host threads without ordering) race; use
 *   spec_verify_sample with a workspace of each caller's own for those.
 *   Errors: as spec_verify_sample (without SPEC_ERR_WORKSPACE), SPEC_ERR_SCRATCH as above, and
 *   SPEC_ERR_HIP if the device or the array's address cannot be obtained. */
int spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                               const int32_t* draft_tokens, const float* uniforms,
                               const int32_t* kv_len_in, int B, int K, int V, float temperature,
                               int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len,
                               float* out_p, float* out_q, hipStream_t stream);

/* spec_verify_sample plus the outcome keys of every slot, computed from the same pass over the
 * draft rows ([SSD] section "1. Outcome Prediction": the keys are the draft's top logits; reading
 * the draft rows once for both saves the separate pass of spec_predict_outcomes).
 * Results of the verification are identical to spec_verify_sample's, bit for bit.
 *   F             keys per slot, 1 <= F (+1 when exclude_draft) <= min(SPEC_MAX_F, V);
 *   exclude_draft nonzero: slot k skips the draft token x_k (see spec_predict_fanout);
 *   out_keys      [B,K,F] int32 (required): slot k's F tokens with the largest draft logits,
 *                 ordered by logit descending then id ascending (x_k skipped when asked);
 *   out_key_prob  [B,K,F] float (nullable): q_k(key) at the call's temperature, from the same
 *                 row statistics as out_q.
 * Two launches, as spec_verify_sample: the statistics pass also keeps every draft-row wave's
 * maximum, and the draw's grid has one more workgroup per draft slot that selects the slot's
 * keys while the draw runs (re-reading only the parts of the draft row that can hold a key);
 * errors as for spec_verify_sample, SPEC_ERR_ARG also for F out of range or a null out_keys. */
int spec_verify_sample_keys(const void* target_logits, const void* draft_logits, int dtype,
                            const int32_t* draft_tokens, const float* uniforms,
                            const int32_t* kv_len_in, int B, int K, int V, float temperature,
                            int F, int exclude_draft, int32_t* out_tokens, int32_t* out_tau,
                            int32_t* out_kv_len, float* out_p, float* out_q, int32_t* out_keys,
                            float* out_key_prob, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Verification of a mixed batch: request b at its own temperature temperatures[b] ([SD] stage 3:
 * temperature zero is the argmax rule, a positive temperature the probability-ratio rule).
 *   temperatures [B] float (device): T_b = 0 verifies request b greedily (as spec_verify_greedy:
 *                its draft rows are not read); T_b > 0 by speculative sampling at T_b (as
 *                spec_verify_sample with temperature T_b: same outputs, bit for bit); a T_b that is
 *                negative, not finite, or so small that log2(e)/T_b is not finite is a row error
 *                for request b (the host cannot check device data).
 * Other arguments and outputs as for spec_verify_sample. For a T_b = 0 request out_p[b,k] is 1
 * when x_k is the target's top choice and 0 otherwise, and out_q[b,k] is 1 (a temperature-zero
 * draft puts all its probability on its token). Errors as for spec_verify_sample, without the
 * host-side temperature check; SPEC_ERR_ARG also for a null temperatures. */
int spec_verify_mixed(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* kv_len_in, const float* temperatures, int B, int K, int V,
                      int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len, float* out_p,
                      float* out_q, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Prompt-lookup drafting, a draft source with no draft model ([SD] section
 * "別のドラフトモデルは常に必要なのか?", the n-gram and prompt-search bullet: match the latest
 * text against the prompt and the output so far, and propose the tokens that followed).
 *   context     [B, ld] int32 (device): row b holds request b's tokens so far, prompt then
 *               output; only the first context_len[b] are read. Token ids are compared only.
 *   ld          row stride in tokens, 1 <= ld <= SPEC_MAX_CONTEXT.
 *   context_len [B] int32 (device): L_b; a value outside [0, ld] is a row error.
 *   n_max, n_min  span lengths tried, 1 <= n_min <= n_max <= SPEC_MAX_NGRAM.
 *   K           tokens drafted at most, 1 <= K <= SPEC_MAX_K.
 * Rule: for n = min(n_max, L-1) down to n_min, the span ctx[L-n:] is looked for at earlier
 * starts j <= L-n-1; the first n with an occurrence is used, at its largest j. The draft is
 * ctx[src : src + len], src = j + n, len = min(K, L - src) >= 1; with no occurrence, len = 0.
 * Outputs (device): out_tokens [B, K] int32 (the draft, -1 past len); out_len [B] int32 (len;
 * -1 for a row error); out_ngram [B] int32 (nullable: the n used, 0 without a match);
 * out_src [B] int32 (nullable: src, -1 without a match). One launch, one workgroup per request,
 * no workspace. Errors: SPEC_ERR_ARG for a null required pointer or a size out of range;
 * SPEC_ERR_HIP if the launch fails. */
int spec_ngram_draft(const int32_t* context, long long ld, const int32_t* context_len, int B,
                     int n_max, int n_min, int K, int32_t* out_tokens, int32_t* out_len,
                     int32_t* out_ngram, int32_t* out_src, hipStream_t stream);

/* Verification of drafts that come with no distribution, such as spec_ngram_draft's ([SD]
 * stages 3-4 and the closing remark of the section on drafting without a draft model: whatever
 * proposes the candidates, the target checks them with its own distribution). The proposer is
 * taken to put all its probability on its token: q_k is a point mass at x_k.
 *   draft_len [B] int32 (device, nullable = K for every request): request b drafts only its
 *             first n_b slots; x_k for k >= n_b is ignored (any value). n_b outside [0, K] is a
 *             row error.
 *   T > 0: slot k < n_b is kept iff uniforms[b,k] < min(1, p_k(x_k)); at the first rejection
 *          m < n_b the token is drawn with uniforms[b,K] by inverse CDF from p_m with x_m
 *          removed (max(0, p_m - q_m)); with all n_b kept, from p_{n_b} (the bonus row).
 *   T = 0: the greedy rule over the first n_b slots; uniforms may be NULL.
 * Target rows past n_b are not read, so a request costs (n_b + 1) * V logits. Outputs as for
 * spec_verify_sample: tokens [B,K+1] (-1 after slot m), tau = m + 1, kv = kv_in + tau;
 * out_p[b,k] = p_k(x_k) (at T = 0 the top-choice indicator) and out_q[b,k] = 1 for k < n_b, NaN
 * for k >= n_b and for row errors. A row error (n_b, or a drafted token outside [0, V)) gives
 * tau = -1, all tokens -1 and kv unchanged. Host errors as for spec_verify_sample; temperature 0
 * is allowed. */
int spec_verify_point(const void* target_logits, int dtype, const int32_t* draft_tokens,
                      const int32_t* draft_len, const float* uniforms, const int32_t* kv_len_in,
                      int B, int K, int V, float temperature, int32_t* out_tokens,
                      int32_t* out_tau, int32_t* out_kv_len, float* out_p, float* out_q,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification, temperature must be exactly 0 ([SD] stage 3 at temperature zero;
 * [D3D] 検証のしくみ③, 検証のまとめ). g_k = argmax_v target_logits[b,k,v] (lowest v on ties);
 * m = first k with draft_tokens[b,k] != g_k (K if none); y = g_m. Same outputs as
 * spec_verify_sample without probabilities. Draft logits are not needed and not read. */
int spec_verify_greedy(const void* target_logits, int dtype, const int32_t* draft_tokens,
                       const int32_t* kv_len_in, int B, int K, int V, float temperature,
                       int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* spec_verify_greedy with the deciders' poll budget, for testing. Results are identical to
 * spec_verify_greedy, bit for bit, whatever the budget is.
 *   wait_polls the chunk workgroups publish their (max, lowest id) and one deciding workgroup
 *              per request, launched after all of them, polls for these at most this many times
 *              per word (a short sleep apart). Negative selects SPEC_DEFAULT_WAIT_POLLS (what
 *              spec_verify_greedy uses). A decider that runs out streams its request's rows
 *              itself, then waits (up to SPEC_DEFAULT_WAIT_POLLS polls per word) for the words it
 *              gave up on and clears them, so the workspace is left as after any other call and
 *              the next call takes the normal path. 0 makes every decider that does not find all
 *              its words already published take that path. Only if a word has still not arrived
 *              after the second wait (its workgroup was dispatched before the decider, so this
 *              does not happen in practice) does the decider mark the workspace: from then on
 *              every greedy call on it streams its rows inside its deciders (same results, more
 *              time) until spec_workspace_init clears the mark. */
int spec_verify_greedy_ex(const void* target_logits, int dtype, const int32_t* draft_tokens,
                          const int32_t* kv_len_in, int B, int K, int V, float temperature,
                          int32_t* out_tokens, int32_t* out_tau, int32_t* out_kv_len,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          int wait_polls);

/* Outcome-key prediction ([SSD] "1. Outcome Prediction"; [D3D] "答え:…").
 * For every request b and slot k < K: out_keys[b,k,0..F-1] = the F token ids with the largest
 * draft_logits[b,k,:], ordered by logit descending then id ascending; a key (k, t) predicts
 * "k drafts kept, target places t". out_key_prob[b,k,f] (nullable) = q_k(key) at T > 0; at
 * T = 0 it is 1 for the first key and 0 for the others. */
int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int K, int V, int F,
                          float temperature, int32_t* out_keys, float* out_key_prob,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Outcome keys with a per-slot fan-out ([D3D] "答え:…": for each of the first P draft positions
 * the drafter prepares candidates for the token the target would place were that position the
 * first rejection, its own 2nd and 3rd choices in the page's setting; [SSD] section 1: how many
 * candidates each position gets is the fan-out).
 *   fanout     HOST array of P ints, 1 <= P <= K: F_k >= 0 keys for slot k (at least one key in
 *              total). F_k <= SPEC_MAX_F, or SPEC_MAX_F - 1 when draft_tokens is given; the F_k
 *              (+1 when draft_tokens is given) must not exceed V.
 *   draft_tokens [B,K] int32 (nullable): when given, slot k skips the draft token x_k. After a
 *              rejection at slot k the target never places x_k (its residual weight is zero;
 *              at temperature zero the placed token differs from x_k by definition), so the
 *              slot's keys are the best tokens that can actually be placed; with greedy drafts
 *              they are the drafter's 2nd, 3rd, ... choices.
 * Slot k's keys are the F_k tokens with the largest draft_logits[b,k,:] (x_k skipped as above),
 * ordered by logit descending then id ascending, written at out_keys[b, off_k .. off_k+F_k),
 * off_k = F_0 + ... + F_{k-1}; out_keys is [B,S] int32 with S = F_0 + ... + F_{P-1}.
 * out_key_prob [B,S] (nullable) = q_k(key) at T > 0; at T = 0, 1 for the row's argmax token
 * (lowest id among equal maxima) and 0 for any other key. Only rows k < P with F_k > 0 are read.
 * The workspace is sized by spec_workspace_bytes(B, K, V, F) for any F. Errors as for
 * spec_predict_outcomes (SPEC_ERR_ARG also for P or fan-outs out of range, or S = 0). */
int spec_predict_fanout(const void* draft_logits, int dtype, const int32_t* draft_tokens, int B,
                        int K, int V, int P, const int32_t* fanout, float temperature,
                        int32_t* out_keys, float* out_key_prob, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* The prepared continuation each verification outcome selects ([D3D] sections "ヒット" and
 * "ミス": a placed token among the prepared candidates is a hit; a placed token outside them, or
 * a rejection beyond the prepared positions, is a miss; section "答え:…": one more continuation
 * is prepared for the case where every draft is kept).
 *   tau [B], tokens [B,K+1] int32 (device): outputs of spec_verify_sample or spec_verify_greedy;
 *   keys [B,S] int32 (device): out_keys of spec_predict_fanout with the same P and fanout (HOST
 *   array, same rules); all_accept: nonzero when a continuation for "every draft kept" exists.
 * out_slot [B] int32 (device): off_m + j when the request kept m = tau-1 < P drafts and placed
 * keys[b, off_m + j]; S when it kept all K drafts (tau = K+1) and all_accept is nonzero; -1
 * otherwise (a miss, or a row error tau = -1). One thread per request; no workspace.
 * Errors: SPEC_ERR_ARG for null pointers, B < 1, K out of [1, SPEC_MAX_K], P out of [1, K] or a
 * fan-out out of [0, SPEC_MAX_F] (or S = 0); SPEC_ERR_HIP for a failed launch. */
int spec_outcome_lookup(const int32_t* tau, const int32_t* tokens, const int32_t* keys, int B,
                        int K, int P, const int32_t* fanout, int all_accept, int32_t* out_slot,
                        hipStream_t stream);

/* Paged KV-cache rewind after a verification round ([SD] section "speculative decodingとKV cache、
 * プロンプトキャッシュの関係は?": both models' caches are truncated past the kept entries).
 * Call once per cache (target and draft caches have their own tables and lengths).
 *   block_tables [B, max_blocks] int32 (device, read and written): request b's entries [0, L)
 *                live in blocks block_tables[b][0 .. ceil(L / block_size)).
 *   kv_alloc [B] int32 (device): entries the cache holds now (e.g. kv_len_in + K + 1);
 *   kv_new   [B] int32 (device): entries to keep (e.g. out_kv_len of a verify call; an engine
 *                whose cache lacks the placed token's entry passes one less).
 * The whole blocks [ceil(kv_new / block_size), ceil(kv_alloc / block_size)) (clamped to
 * max_blocks; none when kv_new >= kv_alloc; negative lengths count as 0) are released: their
 * table entries become -1 and their ids are written to out_freed [B * max_blocks] int32 request
 * by request, each request's in table order, from out_offsets[b]; out_offsets [B+1] int32,
 * out_offsets[B] = total released. Deterministic. One workgroup; no workspace.
 * Errors: SPEC_ERR_ARG for null pointers, B < 1, max_blocks < 1, block_size < 1 or
 * B * max_blocks >= 2^31; SPEC_ERR_HIP for a failed launch. */
int spec_kv_rewind(int32_t* block_tables, int B, int max_blocks, int block_size,
                   const int32_t* kv_alloc, const int32_t* kv_new, int32_t* out_freed,
                   int32_t* out_offsets, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
