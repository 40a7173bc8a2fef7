"""A library call reports the status of its own launches only.

An error that an earlier, unrelated runtime call left pending in the HIP
runtime's last-error slot (here: hipSetDevice with an ordinal past the device
count, refused on the host) must not be reported as the library's failure: each
launch's status comes from hipLaunchKernel itself.  The pending error is cleared
at the end so that later launch checks (torch's included) do not see it.
"""
import ctypes

import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import binding, inputs
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

HIP_ERROR_INVALID_DEVICE = 101


def hip_runtime():
    """The HIP runtime this process uses (torch's; the library binds to the same one)."""
    gh.cuda()
    return ctypes.CDLL("libamdhip64.so.7")


def test_a_pending_runtime_error_is_not_reported_as_the_call_s():
    torch = gh.cuda()
    hip = hip_runtime()
    w = inputs.custom("pending", "bf16", 1, 2, 130, 64, True, seed=3)
    x = inputs.generate(w)
    q, k, v, _ = gh.to_device(x)
    torch.cuda.synchronize()
    try:
        assert hip.hipSetDevice(1 << 20) == HIP_ERROR_INVALID_DEVICE
        assert hip.hipPeekAtLastError() == HIP_ERROR_INVALID_DEVICE
        o, lse = torch.empty_like(q), torch.empty((1, 2, 130), dtype=torch.float32, device="cuda")
        binding.fa_fwd_bf16(q, k, v, o, lse, True, w.scale, None)           # one launch
        ws = torch.empty(binding.fa_unfused_workspace_bytes(1, 2, 130, 2), dtype=torch.uint8, device="cuda")
        o2, lse2 = torch.empty_like(q), torch.empty_like(lse)
        binding.fa_fwd_unfused_bf16(q, k, v, o2, lse2, True, w.scale, None, ws)   # three launches
        assert hip.hipDeviceSynchronize() == 0
    finally:
        hip.hipGetLastError()  # clear what the test left pending
    assert hip.hipPeekAtLastError() == 0
    ro, rl = oracle.attention(x.q, x.k, x.v, True, w.scale, None, nthreads=gh.oracle_threads())
    for a, b in ((o, lse), (o2, lse2)):
        gh.compare("bf16", a.float().cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64), ro, rl,
                   "after a pending runtime error")
