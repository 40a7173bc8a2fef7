"""Test-side fp64 blockwise online-softmax attention (a pin for the oracle, not an oracle).

Written from the loop the pages describe: the outer loop walks query blocks,
the inner loop walks key/value blocks, and per block the running row max m,
the running sum l and the unnormalised output O are re-based to the new max
and extended; O is divided by l once at the end and L = m + log(l) is kept per
row ("GPU 与 TPU：让硬件不再是黑魔法" §11.3-§11.4; "FlashAttention 1–4: How
IO-Awareness Reshaped the Attention Kernel", sections "FlashAttention (v1)" and
"FlashAttention-2").  Added here, because the configurations need them: the
additive -inf mask (causal and per-row key limits), and the guard that keeps a
fully masked row from computing -inf minus -inf ("07 GPU、资源估算与
FlashAttention" §7.8).

``stale_threshold`` > 0 gives the conditional-rescaling variant of
"FlashAttention 1–4 ...", section "FlashAttention-4": the reference max only
moves when a block's max exceeds it by more than the threshold (natural-log
units here), which leaves O / l unchanged.

Used only to check that the oracle's result does not depend on how the rows
are split into blocks.  Shares no code with the oracle or the HIP path.
"""
from __future__ import annotations

import numpy as np


def mask_matrix(N: int, causal: bool, limits) -> np.ndarray:
    """Boolean [N, N] matrix of valid (query i, key j) pairs for one batch item."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    ok = np.ones((N, N), bool)
    if causal:
        ok &= j <= i
    if limits is not None:
        ok &= j < np.asarray(limits)[:, None]
    return ok


def online_attention(q, k, v, causal=False, scale=None, kv_limit=None,
                     block_q=128, block_k=128, stale_threshold=0.0):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o_out = np.zeros_like(q)
    lse_out = np.zeros((B, H, N))
    for b in range(B):
        valid = mask_matrix(N, causal, None if kv_limit is None else kv_limit[b])
        for h in range(H):
            for i0 in range(0, N, block_q):
                qi = q[b, h, i0:i0 + block_q]
                rows = qi.shape[0]
                m = np.full(rows, -np.inf)
                l = np.zeros(rows)
                acc = np.zeros((rows, d))
                for j0 in range(0, N, block_k):
                    s = (qi @ k[b, h, j0:j0 + block_k].T) * scale
                    s = np.where(valid[i0:i0 + block_q, j0:j0 + block_k], s, -np.inf)
                    block_max = s.max(axis=1)
                    if stale_threshold > 0:
                        move = (block_max > m + stale_threshold) | np.isneginf(m)
                        m_new = np.where(move, np.maximum(m, block_max), m)
                    else:
                        m_new = np.maximum(m, block_max)
                    # guard: a row with no valid key so far keeps a finite reference
                    ref = np.where(np.isneginf(m_new), 0.0, m_new)
                    p = np.exp(s - ref[:, None])
                    alpha = np.exp(np.where(np.isneginf(m), -np.inf, m - ref))
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, j0:j0 + block_k]
                    m = m_new
                pos = l > 0
                o_out[b, h, i0:i0 + rows] = np.where(pos[:, None], acc / np.where(pos, l, 1.0)[:, None], 0.0)
                lse_out[b, h, i0:i0 + rows] = np.where(pos, m + np.log(np.where(pos, l, 1.0)), -np.inf)
    return o_out, lse_out
