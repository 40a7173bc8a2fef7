"""Race check of the forward kernels' LDS pipeline: libfa_single_stage.so holds
the same forward kernels built with one LDS stage (a tile is loaded only after
every wave has finished reading the previous one), and its results must equal
libfa.so's bit for bit -- on ragged sweeps and on full-size workloads, for the
bf16 forward and the FP8 forward (Q given as codes or encoded in the kernel)."""
import numpy as np
import pytest

from flashattention_forward_attn_amd import binding, inputs
from tests.gpu_helpers import cuda, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    cuda()
    return binding.load(), binding.open_library(binding.SINGLE_STAGE_LIBRARY)


def fwd_both(torch, libs, q, k, v, causal, scale, lim):
    B, H, N, d = q.shape
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in libs:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        assert lib.fa_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                               int(causal), scale, None if lim is None else lim.data_ptr(), stream) == 0
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def fp8_both(torch, libs, q, k, v, causal, scale, lim, q_in_kernel=False):
    B, H, N, d = q.shape
    signs = torch.from_numpy(inputs.fp8_signs(d, seed=N)).cuda()
    qc, qe = binding.fp8_quantize(q, signs, binding.FP8_Q_TILE)
    kc, ke = binding.fp8_quantize(k, signs, binding.FP8_K_TILE)
    stream = torch.cuda.current_stream().cuda_stream
    limp = None if lim is None else lim.data_ptr()
    outs = []
    for lib in libs:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        if q_in_kernel:
            st = lib.fa_fwd_fp8_qbf16(q.data_ptr(), signs.data_ptr(), kc.data_ptr(), ke.data_ptr(), v.data_ptr(),
                                      o.data_ptr(), lse.data_ptr(), B, H, N, d, int(causal), scale, limp, stream)
        else:
            st = lib.fa_fwd_fp8(qc.data_ptr(), qe.data_ptr(), kc.data_ptr(), ke.data_ptr(), v.data_ptr(),
                                o.data_ptr(), lse.data_ptr(), B, H, N, d, int(causal), scale, limp, stream)
        assert st == 0
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def fp8q_both(torch, libs, q, k, v, causal, scale, lim):
    return fp8_both(torch, libs, q, k, v, causal, scale, lim, q_in_kernel=True)


def same(outs, what):
    (o1, l1), (o2, l2) = outs
    assert torch_equal(o1, o2), f"{what}: O differs between the pipelined and single-stage builds"
    assert torch_equal(l1, l2), f"{what}: LSE differs between the pipelined and single-stage builds"


def torch_equal(a, b):
    import torch
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("path", ["bf16", "fp8", "fp8q"])
@pytest.mark.parametrize("mask", ["none", "random"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200, 1000])
def test_sweep(libs, N, causal, d, mask, path):
    torch = cuda()
    w = inputs.custom(f"ss_n{N}", "bf16", 2, 3, N, d, causal, seed=N + d)
    x = inputs.generate(w)
    q, k, v, _ = to_device(x)
    lim = None
    if mask == "random":
        lim = torch.from_numpy(inputs.random_kv_limit(w.B, w.N, seed=N, kind="random")).cuda()
    run = {"bf16": fwd_both, "fp8": fp8_both, "fp8q": fp8q_both}[path]
    same(run(torch, libs, q, k, v, causal, w.scale, lim), f"{path} N={N} causal={causal} d={d} mask={mask}")


@pytest.mark.parametrize("path", ["bf16", "fp8", "fp8q"])
@pytest.mark.parametrize("name", ["bf16_causal_b2h32n4096d128", "bf16_keypad_b8h32n1024d128", "bf16_b4h16n2048d64"])
def test_workload(libs, name, path):
    torch = cuda()
    x = inputs.generate(inputs.WORKLOADS[name])
    q, k, v, lim = to_device(x)
    w = x.workload
    run = {"bf16": fwd_both, "fp8": fp8_both, "fp8q": fp8q_both}[path]
    same(run(torch, libs, q, k, v, w.causal, w.scale, lim), f"{path} {name}")
