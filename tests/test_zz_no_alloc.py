"""The no-allocation paged decode, fa_decode_paged_bf16_noalloc, through the C ABI.

It runs the same two kernels as fa_decode_paged_bf16 with the library's static
per-GPU buffer in place of the caller's workspace, so its outputs must equal
that entry point's bit for bit.  Calls come in a row on one GPU: the decode
workload itself (B=64, H=32, d=128, lengths up to 2048), then a smaller one
(B=3, H=2, d=64, lengths 0, 17 and 300), then the first again; the buffer keeps
each call's partials, and no call may depend on what an earlier one left.  The
smaller case is also checked against the oracle.  A call that needs more
scratch than the buffer holds is refused before anything runs, and the calls
take no device memory.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import binding, inputs
from tests import gpu_helpers as gh
from tests.test_decode_gpu import check as check_decode

pytestmark = pytest.mark.gpu

BIG = "decode_b64h32d128_len2048"


def device_case(torch, x):
    dev16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return (dev16(x.q_bits), dev16(x.k_bits), dev16(x.v_bits), torch.from_numpy(x.block_table).cuda(),
            torch.from_numpy(x.seq_lens).cuda())


def both(x, scale, stream=None):
    """(o, lse) of the workspace entry point and of the no-allocation one, as raw bits."""
    torch = gh.cuda()
    q, kc, vc, bt, sl = device_case(torch, x)
    B, H, d = (int(s) for s in q.shape)
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
        outs.append((o, lse))
    ws = torch.empty(binding.fa_decode_workspace_bytes(B, H, d, int(bt.shape[1])), dtype=torch.uint8,
                     device=q.device)
    binding.fa_decode_paged_bf16(q, kc, vc, bt, sl, outs[0][0], outs[0][1], scale, ws, stream)
    binding.fa_decode_paged_bf16_noalloc(q, kc, vc, bt, sl, outs[1][0], outs[1][1], scale, stream)
    torch.cuda.synchronize()
    raw = [(o.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()) for o, lse in outs]
    return raw, outs[1]


def small_case():
    w = inputs.DecodeWorkload("noalloc_small", B=3, H=2, d=64, max_len=300, seed=21)
    return inputs.generate_decode(w, lens=[0, 17, 300])


def test_noalloc_equals_the_workspace_entry_point_on_calls_in_a_row():
    big = inputs.generate_decode(inputs.DECODE_WORKLOADS[BIG])
    w = big.workload
    assert binding.fa_decode_workspace_bytes(w.B, w.H, w.d, w.max_pages) <= binding.FA_DECODE_SCRATCH_BYTES
    small = small_case()
    for name, x in (("big", big), ("small", small), ("big again", big)):
        print(f"no-alloc decode: {name} B={x.workload.B} H={x.workload.H} d={x.workload.d}", flush=True)
        (ref, got), (o, lse) = both(x, x.workload.scale)
        for a, b, what in zip(ref, got, ("o", "lse")):
            assert np.array_equal(a, b), f"{name}: {what} differs from fa_decode_paged_bf16"
        if x is small:
            ro, rl = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.workload.scale,
                                         nthreads=gh.oracle_threads())
            check_decode(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                         "no-alloc decode, small case")


def test_noalloc_on_a_side_stream():
    torch = gh.cuda()
    x = small_case()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        (ref, got), _ = both(x, -0.3, stream=side)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


def test_noalloc_refuses_more_than_its_scratch_and_takes_no_memory():
    torch = gh.cuda()
    B, H, d, max_pages = 64, 32, 128, 257  # 17 splits of 128 floats per (sequence, head): 17.8 MB
    assert binding.fa_decode_workspace_bytes(B, H, d, max_pages) > binding.FA_DECODE_SCRATCH_BYTES
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, H, 16, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bt = torch.zeros((B, max_pages), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.FAError) as e:
        binding.fa_decode_paged_bf16_noalloc(q, kc, vc, bt, sl, o, lse, 0.1)
    assert e.value.status == 9
    # within the limit the same tensors' first 16 pages run; device memory stays as it was
    bt16 = bt[:, :16].contiguous()
    binding.fa_decode_paged_bf16_noalloc(q, kc, vc, bt16, sl, o, lse, 0.1)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        binding.fa_decode_paged_bf16_noalloc(q, kc, vc, bt16, sl, o, lse, 0.1)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    # zero keys and values: every sequence's output is 0, its lse ln 5
    assert torch.all(o == 0).item()
    assert torch.allclose(lse, torch.full_like(lse, float(np.log(5.0))), atol=1e-6)
