"""fp64 CPU oracle for the verification step of speculative sampling.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute anything in
this package: only the tests, the smoke check and the bench's CPU-baseline leg use it. It shares
no code with the HIP library (no kernels, headers, tables or helpers); the seeded input
generators in `synthetic/` are the only code both sides use.

Modules
  reference  vectorised NumPy oracle in float64 (greedy, sampling, outcome prediction with a
             uniform or per-slot fan-out, hit check and prepared-continuation lookup, draft
             budget, paged KV-cache rewind, mixed temperatures, prompt-lookup drafting and
             verification of drafts without a distribution, decision margins, near-tie flags)
  naive      the same rules as literal pure-Python loops (math.exp, running sums), used only to
             cross-check `reference` on tiny inputs

Sources (page titles and sections):
  [SD]   "speculative decodingとは" (lotook.com): section "speculative decodingはどのような手順で
         動くのか?" (the four-stage loop; stage 3 accept/reject, stage 4 residual resample and
         bonus token), section "speculative decodingとKV cache、プロンプトキャッシュの関係は?"
         (KV-cache rewind), section "別のドラフトモデルは常に必要なのか?" (n-gram and prompt
         lookup drafting; the target checks any proposer's candidates with its own distribution)
         and the FAQ entry on output quality (losslessness).
  [SSD]  "Speculative Speculative Decoding (SSD)" (jiwasawa.github.io): section
         "1. Outcome Prediction (The Saguaro Cache)".
  [D3D]  "LLMの生成を5倍速くする「D3D」を図で読む" (animemo.app): sections "検証のしくみ①",
         "検証のしくみ③", "検証のまとめ", "答え:ありうる結果すべてに、先回りして下書きする",
         "パック", "ヒット", "ミス" and the table under "用意を増やせばいい、わけではない".

Pin status: every function is pinned by a CPU test except the parts the pages give no formula
for (Saguaro's fan-out optimiser and Saguaro sampling), which are not implemented here. The
near-tie margins and flags are pinned by hand-worked margins on both sides of the 1e-5 threshold
(accept decisions, bonus and residual draws, the normalisation by the residual mass) and by flag
counts over seeded uniforms against the exact flag probability in closed form; the accept ratio
at tiny temperatures by cases where p and q both underflow.
"""
from .reference import (NEAR_TIE, decode_logits, softmax, log_softmax, residual_weights,
                        inverse_cdf, cdf_margin, accept_ratio, sample_draw_weights,
                        point_draw_weights, draw_weights, point_weights,
                        verify_sample_request, verify_greedy_request, predict_request,
                        verify_sample, verify_greedy, predict_outcomes, outcome_hit,
                        fanout_offsets, predict_fanout_request, predict_fanout, outcome_slot,
                        fanout_budget, kv_rewind, temperature_is_valid, verify_mixed_request,
                        verify_mixed, ngram_draft_request, ngram_draft, verify_point_request,
                        verify_point)

__all__ = ["NEAR_TIE", "decode_logits", "softmax", "log_softmax", "residual_weights",
           "inverse_cdf", "cdf_margin", "accept_ratio", "sample_draw_weights",
           "point_draw_weights", "draw_weights", "point_weights",
           "verify_sample_request", "verify_greedy_request", "predict_request", "verify_sample",
           "verify_greedy", "predict_outcomes", "outcome_hit", "fanout_offsets",
           "predict_fanout_request", "predict_fanout", "outcome_slot", "fanout_budget",
           "kv_rewind", "temperature_is_valid", "verify_mixed_request", "verify_mixed",
           "ngram_draft_request", "ngram_draft", "verify_point_request", "verify_point"]
