"""The library's entry points can be captured in a HIP graph and replayed.

None of them allocates, synchronises or issues a memset, so a caller in a
serving loop can capture them once and replay: here the fused forward, the
backward pass, the paged decode (with and without a workspace) and the FP8
forward are each captured on
torch's capture stream, replayed several times with eager work and
synchronisation in between (the inputs change between replays), and every
replay is compared bit for bit with an eager call on the same inputs.
"""
import numpy as np
import pytest

from flashattention_forward_attn_amd import binding, inputs
from tests.gpu_helpers import cuda

pytestmark = pytest.mark.gpu

REPLAYS = 3


def bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def capture(torch, fn):
    """Capture fn() (which launches on the current stream) into a graph; warm up eagerly first."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_compare(torch, g, refill, eager, outs):
    for r in range(REPLAYS):
        refill(r)
        torch.cuda.synchronize()
        _ = torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        want = eager()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r} differs from eager"


def test_forward_and_backward_graph():
    torch = cuda()
    w = inputs.custom("graph_fwd", "bf16", 2, 3, 300, 128, True, seed=4)
    base = inputs.generate(w)
    q, k, v = (bf16(torch, b) for b in (base.q_bits, base.k_bits, base.v_bits))
    g_out = bf16(torch, inputs.grad_output(w).dout_bits)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(binding.fa_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        binding.fa_fwd_bf16(q, k, v, o, lse, True, w.scale, None, s)
        binding.fa_bwd_bf16(q, k, v, o, g_out, lse, dq, dk, dv, True, w.scale, None, ws, s)

    graph = capture(torch, step)

    def refill(r):
        x = inputs.generate(w, seed=100 + r)
        for dst, bits in ((q, x.q_bits), (k, x.k_bits), (v, x.v_bits)):
            dst.copy_(bf16(torch, bits))

    def eager():
        o2, lse2 = binding.attention(q, k, v, causal=True, scale=w.scale)
        grads = binding.attention_backward(q, k, v, o2, lse2, g_out, causal=True, scale=w.scale)
        return [o2, lse2, *grads]

    replay_and_compare(torch, graph, refill, eager, [o, lse, dq, dk, dv])


def test_decode_graph():
    torch = cuda()
    w = inputs.DecodeWorkload("graph_dec", 6, 4, 128, 700, seed=5)
    x = inputs.generate_decode(w)
    q, kc, vc = bf16(torch, x.q_bits), bf16(torch, x.k_bits), bf16(torch, x.v_bits)
    bt = torch.from_numpy(x.block_table).cuda()
    sl = torch.from_numpy(x.seq_lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(binding.fa_decode_workspace_bytes(w.B, w.H, w.d, w.max_pages), dtype=torch.uint8, device="cuda")

    graph = capture(torch, lambda: binding.fa_decode_paged_bf16(q, kc, vc, bt, sl, o, lse, w.scale, ws,
                                                               torch.cuda.current_stream()))

    def refill(r):  # new queries and new lengths each replay, as a decode loop would have
        rng = np.random.default_rng(r)
        q.copy_(bf16(torch, inputs.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))))
        sl.copy_(torch.from_numpy(rng.integers(0, w.max_len + 1, size=w.B).astype(np.int32)))

    def eager():
        return list(binding.decode_paged(q, kc, vc, bt, sl, scale=w.scale))

    replay_and_compare(torch, graph, refill, eager, [o, lse])


def test_decode_noalloc_graph():
    """The no-allocation decode, the entry point meant for captured loops: every
    replay equals the workspace entry point's eager result."""
    torch = cuda()
    w = inputs.DecodeWorkload("graph_dec_na", 5, 4, 64, 900, seed=8)
    x = inputs.generate_decode(w)
    q, kc, vc = bf16(torch, x.q_bits), bf16(torch, x.k_bits), bf16(torch, x.v_bits)
    bt = torch.from_numpy(x.block_table).cuda()
    sl = torch.from_numpy(x.seq_lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")

    graph = capture(torch, lambda: binding.fa_decode_paged_bf16_noalloc(q, kc, vc, bt, sl, o, lse, w.scale,
                                                                       torch.cuda.current_stream()))

    def refill(r):
        rng = np.random.default_rng(50 + r)
        q.copy_(bf16(torch, inputs.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32))))
        sl.copy_(torch.from_numpy(rng.integers(0, w.max_len + 1, size=w.B).astype(np.int32)))

    def eager():
        return list(binding.decode_paged(q, kc, vc, bt, sl, scale=w.scale))

    replay_and_compare(torch, graph, refill, eager, [o, lse])


def test_fp8_graph():
    torch = cuda()
    w = inputs.custom("graph_fp8", "bf16", 1, 4, 260, 128, False, seed=6)
    x = inputs.generate(w)
    q, k, v = (bf16(torch, b) for b in (x.q_bits, x.k_bits, x.v_bits))
    signs = torch.from_numpy(inputs.fp8_signs(w.d)).cuda()
    qc, qe = binding.fp8_quantize(q, signs, binding.FP8_Q_TILE)
    kc, ke = binding.fp8_quantize(k, signs, binding.FP8_K_TILE)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        binding.fa_fp8_quantize_bf16(q, signs, qc, qe, binding.FP8_Q_TILE, s)
        binding.fa_fp8_quantize_bf16(k, signs, kc, ke, binding.FP8_K_TILE, s)
        binding.fa_fwd_fp8(qc, qe, kc, ke, v, o, lse, False, w.scale, None, s)

    graph = capture(torch, step)

    def refill(r):
        xr = inputs.generate(w, seed=200 + r)
        for dst, bits in ((q, xr.q_bits), (k, xr.k_bits), (v, xr.v_bits)):
            dst.copy_(bf16(torch, bits))

    def eager():
        return list(binding.attention_fp8(q, k, v, signs, causal=False, scale=w.scale))

    replay_and_compare(torch, graph, refill, eager, [o, lse])
