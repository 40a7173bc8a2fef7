"""The C ABI library without a GPU: it loads, exports every function include/fa.h
declares, and rejects invalid arguments on the host before any device call.

Every call below is invalid in at least one argument, so nothing is ever
launched: the fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from flashattention_forward_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, well-aligned, non-overlapping device addresses (never dereferenced)
Q, K, V, O, L, M, W = (0x10000000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"fa_fwd_bf16", "fa_fwd_f32", "fa_fwd_unfused_bf16", "fa_fwd_unfused_f32",
            "fa_unfused_workspace_bytes", "fa_status_str"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_single_stage_build_exports_the_same_functions():
    """The race-check build of the forward kernels carries the whole ABI too."""
    other = binding.open_library(binding.SINGLE_STAGE_LIBRARY)
    for name in declared_functions():
        assert hasattr(other, name), name
    assert other.fa_fwd_bf16(None, K, V, O, L, 2, 3, 100, 128, 0, 0.125, None, None) == 1


def test_status_strings(lib):
    for code in range(10):
        s = lib.fa_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_str(99).decode() == "unknown status"


def fwd(lib, name="fa_fwd_bf16", q=Q, k=K, v=V, o=O, l=L, B=2, H=3, N=100, d=128, causal=0, scale=0.125, m=None):
    return getattr(lib, name)(q, k, v, o, l, B, H, N, d, causal, scale, m, None)


@pytest.mark.parametrize("name", ["fa_fwd_bf16", "fa_fwd_f32"])
def test_fused_validation(lib, name):
    assert fwd(lib, name, q=None) == 1
    assert fwd(lib, name, l=None) == 1
    assert fwd(lib, name, B=0) == 2
    assert fwd(lib, name, N=-5) == 2
    assert fwd(lib, name, B=1 << 12, H=1 << 12, N=1 << 8, d=64) == 2  # 2^38 elements
    assert fwd(lib, name, d=96) == 3
    assert fwd(lib, name, d=256) == 3
    assert fwd(lib, name, scale=float("nan")) == 4
    assert fwd(lib, name, scale=float("inf")) == 4
    assert fwd(lib, name, scale=float("-inf")) == 4
    # every finite scale passes (zero and negative too): the next check answers
    assert fwd(lib, name, scale=0.0, q=Q + 8) == 5
    assert fwd(lib, name, scale=-0.0, q=Q + 8) == 5
    assert fwd(lib, name, scale=-0.1, q=Q + 8) == 5
    assert fwd(lib, name, q=Q + 8) == 5
    assert fwd(lib, name, o=O + 2) == 5
    assert fwd(lib, name, l=L + 2) == 5
    assert fwd(lib, name, m=M + 1) == 5
    assert fwd(lib, name, o=Q) == 8            # output over an input
    assert fwd(lib, name, l=K + 64) == 8       # lse inside k
    assert fwd(lib, name, l=O + 16) == 8       # lse inside o
    assert fwd(lib, name, m=O + 1024) == 8     # kv_limit inside o


def unfused(lib, name="fa_fwd_unfused_bf16", ws=W, ws_bytes=None, B=2, H=3, N=100, d=128, **kw):
    elem = 2 if name.endswith("bf16") else 4
    if ws_bytes is None:
        ws_bytes = lib.fa_unfused_workspace_bytes(B, H, N, elem)
    q, k, v, o, l = kw.get("q", Q), kw.get("k", K), kw.get("v", V), kw.get("o", O), kw.get("l", L)
    return getattr(lib, name)(q, k, v, o, l, B, H, N, d, 0, kw.get("scale", 0.125), kw.get("m"), ws, ws_bytes,
                              None)


@pytest.mark.parametrize("name", ["fa_fwd_unfused_bf16", "fa_fwd_unfused_f32"])
def test_unfused_validation(lib, name):
    assert unfused(lib, name, q=None) == 1
    assert unfused(lib, name, d=80) == 3
    assert unfused(lib, name, scale=float("nan")) == 4
    assert unfused(lib, name, scale=-1.0, ws=None) == 6
    assert unfused(lib, name, scale=0.0, ws=None) == 6
    assert unfused(lib, name, ws=None) == 6
    assert unfused(lib, name, ws_bytes=100) == 6
    assert unfused(lib, name, ws=W + 128) == 6        # 256-byte alignment
    assert unfused(lib, name, ws=O) == 8              # workspace over the output
    assert unfused(lib, name, B=300, H=300, N=1, d=64) == 2  # B*H beyond the grid limit
    assert unfused(lib, name, o=K) == 8
    assert unfused(lib, name, B=1, H=1, N=32769, d=64) == 2  # N beyond the unfused limit


def test_workspace_bytes(lib):
    f = lib.fa_unfused_workspace_bytes
    # ld = N rounded up to 64; S fp32 + P (2 or 4 bytes), each part 256-aligned
    assert f(1, 1, 64, 2) == 64 * 64 * 4 + 64 * 64 * 2
    assert f(1, 1, 65, 2) == 65 * 128 * 4 + 65 * 128 * 2
    assert f(1, 16, 16384, 2) == 16 * 16384 * 16384 * 6
    assert f(2, 32, 4096, 4) == 2 * 32 * 4096 * 4096 * 8
    assert f(1, 1, 3, 2) == 768 + 512  # S: 3*64*4 = 768; P: 3*64*2 = 384, rounded up to 512
    assert f(0, 1, 1, 2) == 0 and f(1, 1, 1, 3) == 0


# backward: fake addresses for o, dout, dq, dk, dv beyond the forward's
DO, DQ, DK, DV = (0x10000000 * (i + 8) for i in range(4))


def bwd(lib, q=Q, k=K, v=V, o=O, g=DO, l=L, dq=DQ, dk=DK, dv=DV, ws=W, ws_bytes=None, B=2, H=3, N=100, d=128,
        causal=0, scale=0.125, m=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(B, H, N)
    return lib.fa_bwd_bf16(q, k, v, o, g, l, dq, dk, dv, B, H, N, d, causal, scale, m, ws, ws_bytes, None)


def test_backward_validation(lib):
    assert bwd(lib, g=None) == 1
    assert bwd(lib, dq=None) == 1
    assert bwd(lib, l=None) == 1
    assert bwd(lib, N=0) == 2
    assert bwd(lib, B=1 << 12, H=1 << 12, N=1 << 8, d=64) == 2
    assert bwd(lib, d=32) == 3
    assert bwd(lib, scale=float("nan")) == 4
    assert bwd(lib, scale=-0.5, q=Q + 8) == 5
    assert bwd(lib, scale=0.0, q=Q + 8) == 5
    assert bwd(lib, dk=DK + 8) == 5
    assert bwd(lib, g=DO + 4) == 5
    assert bwd(lib, l=L + 1) == 5
    assert bwd(lib, ws=None) == 6
    assert bwd(lib, ws_bytes=16) == 6
    assert bwd(lib, ws=W + 64) == 6
    assert bwd(lib, dq=Q) == 8                 # gradient over an input
    assert bwd(lib, dv=DK + 256) == 8          # two gradients overlap
    assert bwd(lib, ws=DQ) == 8                # workspace over a gradient
    assert bwd(lib, dk=L + 1024) == 8          # gradient over lse


def test_backward_workspace_bytes(lib):
    f = lib.fa_bwd_workspace_bytes
    # two fp32 statistics per row, each count rounded up to 64
    assert f(1, 1, 64) == 2 * 64 * 4
    assert f(1, 1, 65) == 2 * 128 * 4
    assert f(2, 32, 4096) == 2 * 2 * 32 * 4096 * 4
    assert f(0, 1, 1) == 0 and f(1, 1, 0) == 0


# paged decode: fake addresses past the ones above
QD, KC, VC, BT, SL, OD, LD, WD = (0x10000000 * (i + 20) for i in range(8))


def dec(lib, q=QD, kc=KC, vc=VC, bt=BT, sl=SL, o=OD, l=LD, ws=WD, ws_bytes=None, B=2, H=3, d=128, page=16,
        max_pages=8, num_pages=20, scale=0.125):
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_bytes(B, H, d, max_pages)
    return lib.fa_decode_paged_bf16(q, kc, vc, bt, sl, o, l, B, H, d, page, max_pages, num_pages, scale, ws,
                                    ws_bytes, None)


def test_decode_validation(lib):
    assert dec(lib, q=None) == 1
    assert dec(lib, bt=None) == 1
    assert dec(lib, sl=None) == 1
    assert dec(lib, l=None) == 1
    assert dec(lib, B=0) == 2
    assert dec(lib, H=70000) == 2
    assert dec(lib, page=32) == 2              # pages of 16 tokens only
    assert dec(lib, max_pages=0) == 2
    assert dec(lib, num_pages=0) == 2
    assert dec(lib, max_pages=65535 * 16 + 1) == 2   # more than 65535 splits
    assert dec(lib, d=96) == 3
    assert dec(lib, scale=float("nan")) == 4
    assert dec(lib, scale=0.0, kc=KC + 8) == 5
    assert dec(lib, scale=-2.0, kc=KC + 8) == 5
    assert dec(lib, kc=KC + 8) == 5
    assert dec(lib, o=OD + 2) == 5
    assert dec(lib, bt=BT + 2) == 5
    assert dec(lib, ws=None) == 6
    assert dec(lib, ws_bytes=64) == 6
    assert dec(lib, ws=WD + 128) == 6
    assert dec(lib, o=KC + 4096) == 8          # output inside the key cache
    assert dec(lib, l=BT) == 8                 # lse over the block table
    assert dec(lib, ws=OD) == 8                # workspace over the output
    assert dec(lib, l=OD + 16) == 8            # lse over the output


def decn(lib, q=QD, kc=KC, vc=VC, bt=BT, sl=SL, o=OD, l=LD, B=2, H=3, d=128, page=16, max_pages=8, num_pages=20,
         scale=0.125):
    return lib.fa_decode_paged_bf16_noalloc(q, kc, vc, bt, sl, o, l, B, H, d, page, max_pages, num_pages, scale, None)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode checks what fa_decode_paged_bf16 checks, in the same
    order, then the scratch limit; every case here fails before anything runs."""
    nan = float("nan")
    assert decn(lib, q=None) == 1
    assert decn(lib, l=None) == 1
    assert decn(lib, B=0) == 2
    assert decn(lib, page=32) == 2
    assert decn(lib, max_pages=65535 * 16 + 1) == 2
    assert decn(lib, d=96) == 3
    assert decn(lib, scale=nan) == 4
    assert decn(lib, scale=0.0, kc=KC + 8) == 5
    assert decn(lib, o=OD + 2) == 5
    assert decn(lib, o=KC + 4096) == 8
    assert decn(lib, l=OD + 16) == 8
    # scratch: n = B * H * ceil(max_pages / 16) splits of d floats and a (max, sum)
    # pair, each part padded to 64 floats, within FA_DECODE_SCRATCH_BYTES
    cap = binding.FA_DECODE_SCRATCH_BYTES
    assert lib.fa_decode_workspace_bytes(1, 32263, 128, 16) <= cap < lib.fa_decode_workspace_bytes(1, 32264, 128, 16)
    assert lib.fa_decode_workspace_bytes(1, 63550, 64, 16) <= cap < lib.fa_decode_workspace_bytes(1, 63551, 64, 16)
    assert decn(lib, B=1, H=32264, max_pages=16, o=OD + 2) == 5       # sizes pass, alignment fails next
    assert decn(lib, B=1, H=32264, max_pages=16) == 9
    assert decn(lib, B=64, H=32, max_pages=257) == 9                    # 17 splits of 128 floats
    assert decn(lib, B=1, H=63551, d=64, max_pages=16) == 9
    assert decn(lib, B=1, H=32263, max_pages=16, o=OD + 2) == 5         # within the limit: next check fails


def test_decode_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.FA_DECODE_SCRATCH_BYTES


def test_decode_workspace_bytes(lib):
    f = lib.fa_decode_workspace_bytes
    # per (sequence, head, 256-key split): d floats, then a (max, sum) pair; each part padded to 64 floats
    assert f(1, 1, 128, 16) == (128 + 64) * 4             # 16 pages = one split
    assert f(1, 1, 128, 17) == (2 * 128 + 64) * 4         # 17 pages = two splits
    assert f(2, 32, 128, 128) == (2 * 32 * 8 * 128 + 2 * 32 * 8 * 2) * 4
    assert f(1, 1, 64, 1) == (64 + 64) * 4
    assert f(0, 1, 128, 1) == 0 and f(1, 1, 96, 1) == 0 and f(1, 1, 128, 0) == 0


# FP8: fake addresses past the ones above
XQ, SG, CQ, EQ, CK, EK, VF, OF, LF = (0x10000000 * (i + 40) for i in range(9))


def quant(lib, x=XQ, sg=SG, c=CQ, e=EQ, B=2, H=3, N=100, d=128, tile=32):
    return lib.fa_fp8_quantize_bf16(x, sg, c, e, B, H, N, d, tile, None)


def fwd8(lib, qc=CQ, qe=EQ, kc=CK, ke=EK, v=VF, o=OF, l=LF, B=2, H=3, N=100, d=128, causal=0, scale=0.125, m=None):
    return lib.fa_fwd_fp8(qc, qe, kc, ke, v, o, l, B, H, N, d, causal, scale, m, None)


def fwd8q(lib, q=XQ, sg=SG, kc=CK, ke=EK, v=VF, o=OF, l=LF, B=2, H=3, N=100, d=128, causal=0, scale=0.125, m=None):
    return lib.fa_fwd_fp8_qbf16(q, sg, kc, ke, v, o, l, B, H, N, d, causal, scale, m, None)


def test_fp8_qbf16_validation(lib):
    assert fwd8q(lib, q=None) == 1
    assert fwd8q(lib, sg=None) == 1
    assert fwd8q(lib, ke=None) == 1
    assert fwd8q(lib, N=0) == 2
    assert fwd8q(lib, B=1, H=1, N=1 << 24, d=128) == 2      # one head past 4 GiB
    assert fwd8q(lib, d=96) == 3
    assert fwd8q(lib, scale=float("nan")) == 4
    assert fwd8q(lib, scale=-3.0, q=XQ + 8) == 5
    assert fwd8q(lib, q=XQ + 8) == 5
    assert fwd8q(lib, sg=SG + 8) == 5          # signs are read 16 bytes at a time
    assert fwd8q(lib, kc=CK + 4) == 5
    assert fwd8q(lib, l=LF + 2) == 5
    assert fwd8q(lib, o=XQ) == 8               # output over q
    assert fwd8q(lib, o=SG) == 8               # output over the signs
    assert fwd8q(lib, l=OF + 64) == 8          # lse over the output


def test_fp8_validation(lib):
    assert quant(lib, sg=None) == 1
    assert quant(lib, e=None) == 1
    assert quant(lib, N=0) == 2
    assert quant(lib, tile=16) == 2          # tiles of 32 (q) or 64 (k) rows only
    assert quant(lib, d=96) == 3
    assert quant(lib, x=XQ + 2) == 5
    assert quant(lib, c=CQ + 8) == 5
    assert quant(lib, e=EQ + 2) == 5
    assert quant(lib, c=XQ + 64) == 8         # codes over the input
    assert quant(lib, e=CQ + 4) == 8          # exponents over the codes
    assert fwd8(lib, qe=None) == 1
    assert fwd8(lib, N=0) == 2
    assert fwd8(lib, d=32) == 3
    assert fwd8(lib, scale=float("inf")) == 4
    assert fwd8(lib, scale=-1.0, kc=CK + 4) == 5
    assert fwd8(lib, scale=0.0, kc=CK + 4) == 5
    assert fwd8(lib, kc=CK + 4) == 5
    assert fwd8(lib, ke=EK + 1) == 5
    assert fwd8(lib, o=VF) == 8               # output over an input
    assert fwd8(lib, l=OF + 64) == 8          # lse over the output


def test_size_limits(lib):
    """Tensors above 2^31 elements pass the shape check (offsets are 64-bit); the
    limits are one head below 4 GiB and fewer than 2^23 tiles of 32 rows.  An
    accepted size returns the next check's error (scale, then alignment), so
    nothing is launched."""
    nan = float("nan")
    big = dict(B=1, H=3, N=1 << 23, d=128)                      # 3 * 2^30 elements per tensor
    assert fwd(lib, scale=nan, **big) == 4
    assert fwd(lib, "fa_fwd_f32", scale=nan, B=1, H=5, N=1 << 22, d=128) == 4   # 5 * 2^29
    assert bwd(lib, scale=nan, **big) == 4
    assert fwd8(lib, scale=nan, **big) == 4
    assert quant(lib, x=XQ + 2, **big) == 5
    # one head: N * d * bytes must stay below 2^32
    assert fwd(lib, scale=nan, B=1, H=1, N=(1 << 24) - 1, d=128) == 4
    assert fwd(lib, scale=nan, B=1, H=1, N=1 << 24, d=128) == 2
    assert fwd(lib, "fa_fwd_f32", scale=nan, B=1, H=1, N=(1 << 23) - 1, d=128) == 4
    assert fwd(lib, "fa_fwd_f32", scale=nan, B=1, H=1, N=1 << 23, d=128) == 2
    assert bwd(lib, scale=nan, B=1, H=1, N=1 << 24, d=128) == 2
    assert fwd8(lib, scale=nan, B=1, H=1, N=1 << 24, d=128) == 2
    assert quant(lib, x=XQ + 2, B=1, H=1, N=1 << 24, d=128) == 2
    # grid: B * H * ceil(N / 32) < 2^23 tiles of 32 rows
    assert fwd(lib, scale=nan, B=1, H=(1 << 23) - 1, N=1, d=64) == 4
    assert fwd(lib, scale=nan, B=1, H=1 << 23, N=1, d=64) == 2
    assert fwd(lib, scale=nan, B=2, H=(1 << 21) - 1, N=33, d=64) == 4
    assert fwd(lib, scale=nan, B=2, H=1 << 21, N=33, d=64) == 2
    assert bwd(lib, scale=nan, B=1 << 12, H=1 << 11, N=32, d=64) == 2
    assert fwd8(lib, scale=nan, B=1 << 12, H=1 << 11, N=32, d=64) == 2
    assert quant(lib, x=XQ + 2, B=1 << 12, H=1 << 11, N=32, d=64) == 2
    # decode: 256 threads per (sequence, head) in one grid dimension
    assert dec(lib, scale=nan, B=65535, H=256) == 4
    assert dec(lib, scale=nan, B=65535, H=257) == 2
