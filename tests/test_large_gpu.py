"""Tensors of more than 2^31 elements on every [B, H, N, d] entry point.

Shape B=2, H=8256, N=1024, d=128: 2.16e9 elements, 4.3 GB per bf16 tensor
(8.7 GB in fp32).  Only four (batch, head) pairs hold data
(inputs.generate_large), two of them starting past element 2^31, and every row
sees the first 64 keys.  Those heads are compared with the oracle run on just
them (the same rows, keys and key limit, hence the same numbers); every other
head is all zeros, so its results are known exactly: O = 0 and LSE = ln 64
(64 equal scores of 0), all gradients 0, FP8 codes 0.  Tolerances are the ones
of the corresponding small-size tests.
"""
import math

import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import binding, inputs
from tests.gpu_helpers import cuda, oracle_threads

pytestmark = pytest.mark.gpu

CASE = inputs.LargeCase()
MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 2e-2           # bf16 forward
F32_REL = 1e-5                                           # fp32 forward, normwise
G_MAX_REL, G_MAX_FLOOR, G_MEAN_REL, G_MEAN_FLOOR = 2e-2, 1e-4, 2.5e-2, 1e-5   # backward


@pytest.fixture(scope="module")
def data():
    assert CASE.elements() > 2 ** 31
    assert CASE.heads[-1] * CASE.N * CASE.d >= 2 ** 31
    return inputs.generate_large(CASE)


@pytest.fixture(autouse=True)
def release():
    yield
    torch = cuda()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def place(torch, bits, dtype):
    """A zero [B, H, N, d] device tensor of `dtype` with the listed heads filled."""
    c = CASE
    t = torch.zeros((c.B * c.H, c.N, c.d), dtype=dtype, device="cuda")
    src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda().to(dtype)
    t.index_copy_(0, torch.tensor(c.heads, device="cuda"), src)
    return t.view(c.B, c.H, c.N, c.d)


def heads_of(torch, t):
    """The listed heads of a [B, H, N, ...] device tensor, as float64 numpy [1, S, N, ...]."""
    flat = t.reshape(CASE.B * CASE.H, *t.shape[2:])
    sel = flat.index_select(0, torch.tensor(CASE.heads, device="cuda"))
    return sel.float().cpu().numpy().astype(np.float64)[None]


def others(torch, t):
    """All heads except the listed ones, flattened per head: [B*H - S, ...] on the device."""
    flat = t.reshape(CASE.B * CASE.H, -1)
    keep = torch.ones(CASE.B * CASE.H, dtype=torch.bool, device="cuda")
    keep[list(CASE.heads)] = False
    return flat[keep]


def limits(torch):
    return torch.full((CASE.B, CASE.N), CASE.limit, dtype=torch.int32, device="cuda")


def oracle_limit():
    return np.full((1, CASE.N), CASE.limit, dtype=np.int32)


def check_zero_heads(torch, o, lse):
    assert int(torch.count_nonzero(others(torch, o))) == 0, "O of all-zero heads is not 0"
    rest = others(torch, lse).double()
    assert float((rest - math.log(CASE.limit)).abs().max()) <= 1e-6, "LSE of all-zero heads is not ln 64"


def test_forward_bf16(data):
    torch = cuda()
    q, k, v = (place(torch, getattr(data, n + "_bits"), torch.bfloat16) for n in ("q", "k", "v"))
    o, lse = binding.attention(q, k, v, causal=False, scale=CASE.scale, kv_limit=limits(torch))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data.values("q"), data.values("k"), data.values("v"), causal=False,
                              scale=CASE.scale, kv_limit=oracle_limit(), nthreads=oracle_threads())
    go, gl = heads_of(torch, o), heads_of(torch, lse)
    err = np.abs(go - ro)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    assert np.abs(gl - rl).max() <= LSE_ABS
    check_zero_heads(torch, o, lse)


def test_forward_f32(data):
    torch = cuda()
    q, k, v = (place(torch, getattr(data, n + "_bits"), torch.float32) for n in ("q", "k", "v"))
    o, lse = binding.attention(q, k, v, causal=False, scale=CASE.scale, kv_limit=limits(torch))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(data.values("q"), data.values("k"), data.values("v"), causal=False,
                              scale=CASE.scale, kv_limit=oracle_limit(), nthreads=oracle_threads())
    go, gl = heads_of(torch, o), heads_of(torch, lse)
    assert np.abs(go - ro).max() <= F32_REL * np.abs(ro).max()
    assert np.abs(gl - rl).max() <= F32_REL * np.abs(rl).max()
    check_zero_heads(torch, o, lse)


def test_backward(data):
    """The backward alone: the listed heads' O and LSE are the oracle's (rounded to
    the storage types); dO is zero outside them, so every other gradient is 0."""
    torch = cuda()
    q, k, v, dout = (place(torch, getattr(data, n + "_bits"), torch.bfloat16) for n in ("q", "k", "v", "dout"))
    lim = limits(torch)
    o, lse = binding.attention(q, k, v, causal=False, scale=CASE.scale, kv_limit=lim)
    ro, rl = oracle.attention(data.values("q"), data.values("k"), data.values("v"), causal=False,
                              scale=CASE.scale, kv_limit=oracle_limit(), nthreads=oracle_threads())
    idx = torch.tensor(CASE.heads, device="cuda")
    o16 = torch.from_numpy(ro[0]).to(torch.bfloat16).cuda()
    o.view(CASE.B * CASE.H, CASE.N, CASE.d).index_copy_(0, idx, o16)
    lse.view(CASE.B * CASE.H, CASE.N).index_copy_(0, idx, torch.from_numpy(rl[0]).float().cuda())
    dq, dk, dv = binding.attention_backward(q, k, v, o, lse, dout, causal=False, scale=CASE.scale, kv_limit=lim)
    torch.cuda.synchronize()
    o_st = o16.float().cpu().numpy().astype(np.float64)[None]
    ref = oracle.attention_bwd(data.values("q"), data.values("k"), data.values("v"), data.values("dout"),
                               causal=False, scale=CASE.scale, kv_limit=oracle_limit(), nthreads=oracle_threads(),
                               o=o_st)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        got = heads_of(torch, g)
        err = np.abs(got - r)
        assert err.max() <= G_MAX_REL * np.abs(r).max() + G_MAX_FLOOR, (name, err.max())
        assert err.mean() <= G_MEAN_REL * np.abs(r).mean() + G_MEAN_FLOOR, (name, err.mean())
        assert int(torch.count_nonzero(others(torch, g))) == 0, f"{name} of all-zero heads is not 0"
    for g in (dk, dv):   # keys past the limit get no gradient
        assert np.all(heads_of(torch, g)[:, :, CASE.limit:] == 0.0)


def test_fp8(data):
    torch = cuda()
    q, k, v = (place(torch, getattr(data, n + "_bits"), torch.bfloat16) for n in ("q", "k", "v"))
    signs = inputs.fp8_signs(CASE.d, seed=CASE.seed)
    sd = torch.from_numpy(signs).cuda()
    codes, exps = binding.fp8_quantize(q, sd, binding.FP8_Q_TILE)
    torch.cuda.synchronize()
    rc, re = oracle.fp8_quantize(data.values("q"), signs, tile_rows=32, nthreads=oracle_threads())
    np.testing.assert_array_equal(heads_of(torch, codes).astype(np.int64), rc.astype(np.int64))
    np.testing.assert_array_equal(heads_of(torch, exps).astype(np.int64), re.astype(np.int64))
    zc, ze = oracle.fp8_quantize(np.zeros((1, 1, 32, CASE.d)), signs, tile_rows=32)
    assert int(torch.count_nonzero(others(torch, codes))) == 0
    assert bool((others(torch, exps) == int(ze.reshape(-1)[0])).all())
    del codes, exps
    o, lse = binding.attention_fp8(q, k, v, sd, causal=False, scale=CASE.scale, kv_limit=limits(torch))
    torch.cuda.synchronize()
    kc, ke = oracle.fp8_quantize(data.values("k"), signs, tile_rows=64, nthreads=oracle_threads())
    ro, rl = oracle.attention_fp8(rc, re, 32, kc, ke, 64, data.values("v"), causal=False, scale=CASE.scale,
                                  kv_limit=oracle_limit(), nthreads=oracle_threads())
    go, gl = heads_of(torch, o), heads_of(torch, lse)
    err = np.abs(go - ro)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    assert np.abs(gl - rl).max() <= LSE_ABS
    check_zero_heads(torch, o, lse)


def test_decode_pool_past_2_31():
    """Paged decode whose sequences live in the last pages of a 4.3 GB pool (past
    element 2^31 of each cache), against the oracle on a pool of just those pages."""
    torch = cuda()
    c = inputs.LargeDecodeCase()
    x = inputs.generate_large_decode(c)
    assert int(x.pages.min()) * c.page_elements() >= 2 ** 31
    dev16 = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    caches = []
    for bits in (x.k_bits, x.v_bits):
        t = torch.zeros((c.num_pages, c.H, inputs.DECODE_PAGE, c.d), dtype=torch.bfloat16, device="cuda")
        t.index_copy_(0, torch.from_numpy(x.pages.astype(np.int64)).cuda(), dev16(bits))
        caches.append(t)
    o, lse = binding.decode_paged(dev16(x.q_bits), caches[0], caches[1], torch.from_numpy(x.block_table).cuda(),
                                  torch.from_numpy(x.seq_lens).cuda())
    torch.cuda.synchronize()
    local = {int(p): i for i, p in enumerate(x.pages)}
    table = np.vectorize(lambda p: local.get(int(p), 0))(x.block_table).astype(np.int32)
    f64 = lambda bits: inputs.bf16_to_f32(bits).astype(np.float64)
    ro, rl = oracle.decode_paged(f64(x.q_bits), f64(x.k_bits), f64(x.v_bits), table, x.seq_lens,
                                 nthreads=oracle_threads())
    err = np.abs(o.float().cpu().numpy() - ro)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - rl).max() <= LSE_ABS
