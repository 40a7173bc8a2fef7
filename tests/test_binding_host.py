"""The Python binding checks every tensor argument (dtype, shape, contiguity,
device) before handing its address to the library, so a mismatched tensor
raises instead of letting a kernel read or write memory the caller did not
mean.  Run on the CPU: the checks come before any library call."""
import pytest
import torch

from flashattention_forward_attn_amd import binding

B, H, N, D = 2, 3, 40, 64


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def fwd_args(**over):
    a = dict(q=bf(B, H, N, D), k=bf(B, H, N, D), v=bf(B, H, N, D), o=bf(B, H, N, D),
             lse=torch.zeros(B, H, N), causal=False, scale=0.125, kv_limit=None)
    a.update(over)
    return a


def test_forward_checks():
    f = binding.fa_fwd_bf16
    with pytest.raises(TypeError, match="k must be"):
        f(**fwd_args(k=torch.zeros(B, H, N, D)))                       # fp32 k for the bf16 path
    with pytest.raises(ValueError, match="v must have shape"):
        f(**fwd_args(v=bf(B, H, N - 1, D)))
    with pytest.raises(ValueError, match="lse must have shape"):
        f(**fwd_args(lse=torch.zeros(B, H, N + 1)))
    with pytest.raises(TypeError, match="kv_limit must be"):
        f(**fwd_args(kv_limit=torch.zeros(B, N, dtype=torch.int64)))
    with pytest.raises(ValueError, match="kv_limit must have shape"):
        f(**fwd_args(kv_limit=torch.zeros(N, B, dtype=torch.int32)))
    with pytest.raises(ValueError, match="o must be contiguous"):
        f(**fwd_args(o=bf(B, H, D, N).transpose(2, 3)))
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        f(**fwd_args())                                                  # right in every way but the device
    with pytest.raises(ValueError, match=r"\[B, H, N, d\]"):
        f(**fwd_args(q=bf(B, N, D)))
    with pytest.raises(TypeError, match="q must be"):
        binding.fa_fwd_f32(**fwd_args())                                 # bf16 tensors for the fp32 path


def test_unfused_and_backward_checks():
    with pytest.raises(TypeError, match="workspace must be"):
        binding.fa_fwd_unfused_bf16(**fwd_args(), workspace=torch.zeros(16))
    g = dict(dout=bf(B, H, N, D), dq=bf(B, H, N, D), dk=bf(B, H, N, D), dv=bf(B, H, N, D))
    a = fwd_args()
    args = [a["q"], a["k"], a["v"], a["o"], g["dout"], a["lse"], g["dq"], g["dk"], g["dv"]]
    with pytest.raises(ValueError, match="dk must have shape"):
        binding.fa_bwd_bf16(*args[:7], bf(B, H, N, D // 2), args[8], False, 0.125)
    with pytest.raises(TypeError, match="dout must be"):
        binding.fa_bwd_bf16(*args[:4], torch.zeros(B, H, N, D), *args[5:], False, 0.125)
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        binding.fa_bwd_bf16(*args, False, 0.125)


def test_decode_checks():
    P, MP = 10, 4
    a = dict(q=bf(B, H, D), k_cache=bf(P, H, 16, D), v_cache=bf(P, H, 16, D),
             block_table=torch.zeros(B, MP, dtype=torch.int32), seq_lens=torch.zeros(B, dtype=torch.int32),
             o=bf(B, H, D), lse=torch.zeros(B, H), scale=0.125)
    with pytest.raises(ValueError, match="v_cache must have shape"):
        binding.fa_decode_paged_bf16(**{**a, "v_cache": bf(P - 1, H, 16, D)})
    with pytest.raises(TypeError, match="seq_lens must be"):
        binding.fa_decode_paged_bf16(**{**a, "seq_lens": torch.zeros(B, dtype=torch.int64)})
    with pytest.raises(ValueError, match="o must have shape"):
        binding.fa_decode_paged_bf16(**{**a, "o": bf(B, H, D, 1)})
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        binding.fa_decode_paged_bf16(**a)


def test_fp8_checks():
    x = bf(B, H, N, D)
    signs = torch.ones(D, dtype=torch.int8)
    codes = torch.zeros(B, H, N, D, dtype=torch.uint8)
    exps = torch.zeros(B, H, 2, dtype=torch.int32)                       # ceil(40 / 32)
    with pytest.raises(ValueError, match="tile_rows"):
        binding.fa_fp8_quantize_bf16(x, signs, codes, exps, 16)
    with pytest.raises(ValueError, match="exps must have shape"):
        binding.fa_fp8_quantize_bf16(x, signs, codes, exps, 64)        # 64-row tiles need 1 exponent per head
    with pytest.raises(TypeError, match="signs must be"):
        binding.fa_fp8_quantize_bf16(x, signs.float(), codes, exps, 32)
    ke = torch.zeros(B, H, 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="k_exps must have shape"):
        binding.fa_fwd_fp8(codes, exps, codes, exps, x, bf(B, H, N, D), torch.zeros(B, H, N), False, 0.125)
    with pytest.raises(ValueError, match="q_codes must be a GPU tensor"):
        binding.fa_fwd_fp8(codes, exps, codes, ke, x, bf(B, H, N, D), torch.zeros(B, H, N), False, 0.125)


def test_fp8_qbf16_checks():
    q = bf(B, H, N, D)
    signs = torch.ones(D, dtype=torch.int8)
    kc = torch.zeros(B, H, N, D, dtype=torch.uint8)
    ke = torch.zeros(B, H, 1, dtype=torch.int32)                         # ceil(40 / 64)
    out = (bf(B, H, N, D), torch.zeros(B, H, N))
    with pytest.raises(TypeError, match="signs must be"):
        binding.fa_fwd_fp8_qbf16(q, signs.to(torch.int32), kc, ke, q, *out, False, 0.125)
    with pytest.raises(ValueError, match="k_exps must have shape"):
        binding.fa_fwd_fp8_qbf16(q, signs, kc, torch.zeros(B, H, 2, dtype=torch.int32), q, *out, False, 0.125)
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        binding.fa_fwd_fp8_qbf16(q, signs, kc, ke, q, *out, False, 0.125)


def test_one_hip_runtime_whatever_loads_first():
    """A fresh process that calls into the library before importing torch maps one
    HIP runtime, the one torch uses: the binding imports torch before it opens the
    library.  (torch's HIP library asks for its bundled runtime by file name, so the
    other order would map the system runtime and then torch's beside it.)"""
    import os
    import subprocess
    import sys
    code = (
        "from flashattention_forward_attn_amd import binding\n"
        "binding.fa_decode_workspace_bytes(1, 1, 128, 1)\n"
        "import torch\n"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(paths), *sorted(paths))\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    count, *paths = out.stdout.split()
    assert int(count) == 1, paths
    assert os.path.dirname(paths[0]) == os.path.join(os.path.dirname(torch.__file__), "lib"), paths
