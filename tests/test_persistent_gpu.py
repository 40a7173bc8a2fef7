"""The bf16 forward's walk over query blocks.

Without a key limit, one workgroup per CU walks several 256-row query blocks
(in rounds, the odd rounds mirrored); with a key limit every block has a
workgroup of its own.  A limit of N for every row removes no key, so the two
launches do the same arithmetic and must agree bit for bit.  The shapes below
have more blocks than the chip has CUs, and their block counts leave the last
round partly empty (some workgroups take one block fewer).  One shape is also
compared with the oracle in full.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import inputs
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

# (B, H, N, d, causal): 300, 280, 514 and 480 query blocks of 256 rows
SHAPES = [(1, 300, 256, 64, False), (1, 300, 256, 64, True), (2, 70, 512, 128, True),
          (1, 257, 300, 128, False), (3, 40, 1000, 64, True)]


def blocks(B, H, N):
    return B * H * -(-N // 256)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}n{}d{}{}".format(*s[:4], "c" if s[4] else ""))
def test_block_walk_matches_one_block_per_workgroup(shape):
    B, H, N, d, causal = shape
    torch = gh.cuda()
    assert blocks(B, H, N) > torch.cuda.get_device_properties(0).multi_processor_count
    x = inputs.generate(inputs.custom("walk", "bf16", B, H, N, d, causal, seed=B * 1000 + H + N + d))
    o_walk, l_walk = gh.run(x)
    o_one, l_one = gh.run(x, kv_limit_override=np.full((B, N), N, np.int32))
    assert np.array_equal(o_walk, o_one), "outputs differ between the two launch forms"
    assert np.array_equal(l_walk, l_one), "LSE differs between the two launch forms"
    assert np.all(np.isfinite(o_walk)) and np.all(np.isfinite(l_walk))


def test_block_walk_against_oracle():
    B, H, N, d, causal = SHAPES[1]
    x = inputs.generate(inputs.custom("walk_oracle", "bf16", B, H, N, d, causal, seed=7))
    o, lse = gh.run(x)
    ro, rl = oracle.attention(x.q, x.k, x.v, causal, x.workload.scale, None, nthreads=gh.oracle_threads())
    gh.compare("bf16", o, lse, ro, rl, "bf16 block walk b1h300n256d64 causal")
