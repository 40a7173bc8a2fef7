"""GPU parity of the paged decode (fa_decode_paged_bf16) against the fp64 oracle.

o and lse are compared with oracle.decode_paged on the same seeded caches, with
the forward's bf16 tolerances (max |o - o_ref| <= 2e-2, mean <= 2e-3 over the
compared elements; lse max-abs <= 2e-2 over sequences with a key; an empty
sequence exactly o = 0, lse = -inf).  The documented handling of cache contents
is checked too: a block-table entry outside the pool reads as a zero page,
slots past a sequence's length do not matter even when they hold NaN bit
patterns, and lengths are clamped to the table.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import binding, inputs
from tests.gpu_helpers import cuda, oracle_threads

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 2e-2


def run(x, block_table=None, seq_lens=None, k_bits=None, v_bits=None):
    torch = cuda()
    dev16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q = dev16(x.q_bits)
    kc = dev16(x.k_bits if k_bits is None else k_bits)
    vc = dev16(x.v_bits if v_bits is None else v_bits)
    bt = torch.from_numpy(np.ascontiguousarray(x.block_table if block_table is None else block_table, np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(x.seq_lens if seq_lens is None else seq_lens, np.int32)).cuda()
    o, lse = binding.decode_paged(q, kc, vc, bt, sl, scale=x.workload.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def reference(x, block_table=None, seq_lens=None, k=None, v=None):
    return oracle.decode_paged(x.q, x.k_cache if k is None else k, x.v_cache if v is None else v,
                               x.block_table if block_table is None else block_table,
                               x.seq_lens if seq_lens is None else seq_lens, scale=x.workload.scale,
                               nthreads=oracle_threads())


def check(o, lse, ro, rl, what):
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty sequences differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty sequence with nonzero output"
    err = np.abs(o - ro)
    assert err.max(initial=0.0) <= MAX_ABS, f"{what}: max err {err.max():.3g}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean err {err.mean():.3g}"
    if (~empty).any():
        lerr = np.abs(lse[~empty] - rl[~empty]).max()
        assert lerr <= LSE_ABS, f"{what}: lse err {lerr:.3g}"


EDGE_LENS = [0, 1, 15, 16, 17, 63, 64, 65, 200, 512]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H", [1, 4])
def test_decode_edge_lengths(d, H):
    w = inputs.DecodeWorkload(f"dec_edges_h{H}_d{d}", len(EDGE_LENS), H, d, 512, seed=d + H)
    x = inputs.generate_decode(w, lens=EDGE_LENS)
    o, lse = run(x)
    ro, rl = reference(x)
    check(o, lse, ro, rl, f"edges H={H} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_decode_random_lengths(d, seed):
    w = inputs.DecodeWorkload(f"dec_rand_{seed}_{d}", 7, 3, d, 1000, seed=seed)
    x = inputs.generate_decode(w)
    o, lse = run(x)
    ro, rl = reference(x)
    check(o, lse, ro, rl, f"random seed={seed} d={d}")


def test_decode_page_outside_pool_reads_zero():
    w = inputs.DecodeWorkload("dec_badpage", 3, 2, 128, 256, seed=7)
    x = inputs.generate_decode(w, lens=[100, 256, 40])
    bt = x.block_table.copy()
    bt[1, 3] = x.num_pages + 5          # inside sequence 1's length, outside the pool
    bt[2, 1] = -7                       # inside sequence 2's length, negative
    o, lse = run(x, block_table=bt)
    # the oracle's view: those logical pages point at an extra all-zero page
    zk = np.concatenate([x.k_cache, np.zeros_like(x.k_cache[:1])])
    zv = np.concatenate([x.v_cache, np.zeros_like(x.v_cache[:1])])
    bt_ref = bt.copy()
    bt_ref[1, 3] = bt_ref[2, 1] = x.num_pages
    ro, rl = reference(x, block_table=bt_ref, k=zk, v=zv)
    check(o, lse, ro, rl, "page outside the pool")


def test_decode_slots_past_length_are_ignored():
    w = inputs.DecodeWorkload("dec_tail", 4, 2, 64, 128, seed=8)
    x = inputs.generate_decode(w, lens=[5, 17, 100, 127])
    kb, vb = x.k_bits.copy(), x.v_bits.copy()
    for b, n in enumerate(x.seq_lens):
        last = x.block_table[b, (int(n) - 1) // 16]
        kb[last, :, int(n) % 16 or 16:, :] = 0x7FC0      # NaN
        vb[last, :, int(n) % 16 or 16:, :] = 0xFF80      # -inf
    o, lse = run(x, k_bits=kb, v_bits=vb)
    ro, rl = reference(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    check(o, lse, ro, rl, "NaN past the length")


def test_decode_length_clamping():
    w = inputs.DecodeWorkload("dec_clamp", 3, 2, 128, 64, seed=9)
    x = inputs.generate_decode(w, lens=[64, 10, 64])
    o, lse = run(x, seq_lens=np.array([64 + 100, -3, 64], np.int32))
    ro, rl = reference(x, seq_lens=np.array([64, 0, 64], np.int32))
    check(o, lse, ro, rl, "clamped lengths")


@pytest.mark.parametrize("name", sorted(inputs.DECODE_WORKLOADS))
def test_decode_workload(name):
    """Full-size decode workloads, every output against the full oracle."""
    x = inputs.generate_decode(inputs.DECODE_WORKLOADS[name])
    o, lse = run(x)
    ro, rl = reference(x)
    check(o, lse, ro, rl, name)


def test_decode_deterministic():
    w = inputs.DecodeWorkload("dec_det", 5, 4, 128, 3000, seed=10)
    x = inputs.generate_decode(w)
    a = run(x)
    b = run(x)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
