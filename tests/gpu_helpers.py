"""Helpers for the GPU parity tests: device copies of seeded inputs, calls
through the C ABI binding, and the comparison against the oracle.

Tolerances (floating point):
  bf16 inputs, fp32 accumulation: max |O - O_ref| <= 2e-2 and mean |O - O_ref| <= 2e-3
    over the compared elements; LSE max-abs <= 2e-2 over rows with a valid key.
  fp32: normwise relative, max |dO| <= 1e-5 * max |O_ref|, and the same for LSE.
  Rows with no valid key must be exact: O == 0 and LSE == -inf.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from flashattention_forward_attn_amd import binding, inputs

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_REL = 1e-5


def cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()  # must exist on a GPU run: no fallback
    return torch


def to_device(x: inputs.Inputs):
    torch = cuda()
    if x.workload.dtype == "bf16":
        def dev(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = dev(x.q_bits), dev(x.k_bits), dev(x.v_bits)
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x.q, x.k, x.v))
    lim = None if x.kv_limit is None else torch.from_numpy(x.kv_limit).cuda()
    return q, k, v, lim


def run(x: inputs.Inputs, unfused: bool = False, kv_limit_override=None):
    """Run the HIP path on x's inputs; returns (o, lse) as float64 numpy arrays."""
    torch = cuda()
    q, k, v, lim = to_device(x)
    if kv_limit_override is not None:
        lim = torch.from_numpy(np.ascontiguousarray(kv_limit_override, np.int32)).cuda()
    o, lse = binding.attention(q, k, v, causal=x.workload.causal, scale=x.workload.scale, kv_limit=lim,
                               unfused=unfused)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(dtype: str, o, lse, o_ref, lse_ref, what: str = ""):
    """Assert the tolerances; returns a dict of the measured errors."""
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with no valid key differ"
    assert np.all(o[empty] == 0.0), f"{what}: fully masked rows must be exactly zero"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    full = ~empty
    err = np.abs(o - o_ref)
    lerr = np.abs(lse[full] - lse_ref[full]) if full.any() else np.zeros(1)
    stats = {"max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()) if err.size else 0.0,
             "lse_max_abs": float(lerr.max(initial=0.0))}
    if dtype == "bf16":
        assert stats["max_abs"] <= BF16_MAX_ABS, f"{what}: {stats}"
        assert stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {stats}"
        assert stats["lse_max_abs"] <= BF16_MAX_ABS, f"{what}: {stats}"
    else:
        scale_o = max(np.abs(o_ref).max(initial=0.0), 1e-30)
        scale_l = max(np.abs(lse_ref[full]).max(initial=0.0), 1e-30) if full.any() else 1.0
        stats["rel"] = stats["max_abs"] / scale_o
        stats["lse_rel"] = stats["lse_max_abs"] / scale_l
        assert stats["rel"] <= F32_REL, f"{what}: {stats}"
        assert stats["lse_rel"] <= F32_REL, f"{what}: {stats}"
    return stats


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))
