// Library-level entry points: version, status strings, workspace sizing and initialisation.
#include "api_common.hpp"

namespace sv {
namespace {

__global__ void zero_words_kernel(unsigned* __restrict__ p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

}  // namespace
}  // namespace sv

extern "C" int spec_abi_version(void) { return SPEC_ABI_VERSION; }

extern "C" const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_ARG: return "invalid argument (null pointer, size, alignment or grid limit)";
    case SPEC_ERR_DTYPE: return "unsupported logit dtype (SPEC_F32 or SPEC_BF16)";
    case SPEC_ERR_TEMPERATURE: return "invalid temperature for this entry point";
    case SPEC_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case SPEC_ERR_HIP: return "HIP launch failed";
    case SPEC_ERR_SCRATCH:
      return "sizes need more scratch than spec_verify_sample_noalloc's fixed per-GPU array "
             "(SPEC_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

extern "C" size_t spec_workspace_bytes(int B, int K, int V, int F) {
  if (sv::check_dims(B, K, V) != SPEC_OK || F < 1 || F > SPEC_MAX_F || F > V) return 0;
  return sv::ws_layout(B, K, V, F, 0).total;
}

extern "C" int spec_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // Clears the whole workspace with a fill kernel (no memset node, so the call may also be
  // recorded in a graph). It holds the greedy path's published words and mark; it is small and
  // this runs rarely.
  if (workspace == nullptr || !sv::is_aligned(workspace, 256)) return SPEC_ERR_WORKSPACE;
  const size_t words = workspace_bytes / sizeof(unsigned);
  if (words == 0) return SPEC_ERR_WORKSPACE;
  const size_t blocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
  hipLaunchKernelGGL(sv::zero_words_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<unsigned*>(workspace), words);
  return sv::launch_status();
}
