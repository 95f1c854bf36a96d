"""spec_verify_sample_noalloc, the entry point for callers that cannot allocate a workspace, on
the GPU: through the C ABI (ctypes binding), its outputs equal spec_verify_sample's with a
workspace of its own, bit for bit, and the oracle's by the parity rules, on calls in a row whose
sizes shrink and grow again (the fixed scratch array keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_12_amd as sv
from gpu_helpers import announce, compare_sample, gpu_sample, poisoned, upload
from synthetic import make_workload

pytestmark = pytest.mark.gpu


def noalloc(wl, dev):
    B, K = wl.B, wl.K
    out = dict(tokens=poisoned((B, K + 1), torch.int32), tau=poisoned((B,), torch.int32),
               kv_len=poisoned((B,), torch.int32), p=poisoned((B, K), torch.float32),
               q=poisoned((B, K), torch.float32))
    sv.spec_verify_sample_noalloc(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"],
                                  dev["kv"], float(wl.T), out=out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_noalloc_equals_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sv.load_library()
    # full C3, then a smaller batch and vocabulary, then full C3 again on other inputs
    for cid, rnd, kw in [(3, 70, {}), (3, 71, dict(B=8, V=40000)), (3, 72, {}),
                         (1, 73, dict(B=3))]:
        wl = make_workload(cid, rnd, **kw)
        dev = upload(wl)
        announce(f"no-alloc C{cid} round {rnd} B={wl.B} K={wl.K} V={wl.V}")
        ref = gpu_sample(wl, dev=dev)
        got = noalloc(wl, dev)
        for k in ref:
            assert np.array_equal(ref[k].view(np.int32), got[k].view(np.int32)), k
        n, f, fb = compare_sample(wl, got)
        announce(f"no-alloc: {n} requests equal the workspace call and the oracle ({f} flagged)")


def test_noalloc_rejects_sizes_beyond_its_array():
    """Sizes whose workspace exceeds the array are refused on the host (the pointers below are
    never read), and the next call still works."""
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib = sv.load_library()
    wl = make_workload(3, 74, B=2, V=1000)
    dev = upload(wl)
    p = {k: v.data_ptr() for k, v in dev.items()}
    code = lib.spec_verify_sample_noalloc(p["target"], p["draft"], sv.SPEC_BF16, p["tokens"],
                                          p["uniforms"], None, 1024, 8, 128256, 0.7, p["tokens"],
                                          p["kv"], None, None, None,
                                          torch.cuda.current_stream().cuda_stream)
    assert sv.STATUS[code] == "SPEC_ERR_SCRATCH"
    got = noalloc(wl, dev)
    ref = gpu_sample(wl, dev=dev)
    for k in ref:
        assert np.array_equal(ref[k].view(np.int32), got[k].view(np.int32)), k
