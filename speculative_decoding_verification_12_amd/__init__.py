"""MI355X-native (gfx950) verification step of speculative decoding.

The work runs in hand-written HIP kernels behind the C ABI of libspecverify.so
(include/spec_verify.h); this package is the thin Python binding used by tests and the bench.
Build the library with `python -m speculative_decoding_verification_12_amd.build`.
"""
from ._binding import (EXPORTS, LIB_PATH, SPEC_BF16, SPEC_DEFAULT_WAIT_POLLS, SPEC_F32,
                       SPEC_MAX_CONTEXT, SPEC_MAX_F, SPEC_MAX_K, SPEC_MAX_NGRAM, SPEC_MAX_V,
                       SPEC_NOALLOC_SCRATCH_BYTES, STATUS, SpecVerifyError, hip_runtime, load_library, new_workspace,
                       prepared_greedy, prepared_sample,
                       spec_kv_rewind, spec_ngram_draft, spec_outcome_lookup,
                       spec_predict_fanout, spec_predict_outcomes, spec_verify_greedy,
                       spec_verify_mixed, spec_verify_point, spec_verify_sample,
                       spec_verify_sample_keys, spec_verify_sample_noalloc,
                       spec_workspace_init, status_string, workspace_bytes)

__all__ = ["EXPORTS", "LIB_PATH", "SPEC_BF16", "SPEC_DEFAULT_WAIT_POLLS", "SPEC_F32",
           "SPEC_MAX_CONTEXT", "SPEC_MAX_F", "SPEC_MAX_K", "SPEC_MAX_NGRAM", "SPEC_MAX_V",
           "SPEC_NOALLOC_SCRATCH_BYTES", "STATUS", "SpecVerifyError", "hip_runtime", "load_library", "new_workspace",
           "prepared_greedy", "prepared_sample",
           "spec_kv_rewind", "spec_ngram_draft", "spec_outcome_lookup", "spec_predict_fanout",
           "spec_predict_outcomes", "spec_verify_greedy", "spec_verify_mixed",
           "spec_verify_point", "spec_verify_sample", "spec_verify_sample_keys",
           "spec_verify_sample_noalloc", "spec_workspace_init", "status_string", "workspace_bytes"]
