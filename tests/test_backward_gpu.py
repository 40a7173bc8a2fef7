"""GPU parity of the backward pass (fa_bwd_bf16) against the fp64 oracle.

The gradients dQ, dK, dV of sum(dO * O) are compared with oracle.attention_bwd
(the chain rule written out, pinned against finite differences of the forward
oracle).  Two kinds of check:

  - parity of the backward alone: the O and LSE handed to the HIP backward are
    the oracle's, rounded to the storage types (bf16, fp32), and the reference
    is the oracle given that same O.  The backward forms its row term
    D_i = <dO_i, O_i> from the O it is handed, so this compares like with like
    on every workload;
  - end to end: the HIP forward's O and LSE feed the HIP backward, against the
    exact gradients.  Here the bf16 rounding of O enters dQ and dK through D.
    On the workload whose scores are scaled by 8 the rows are nearly one-hot
    and that rounding alone (computed by the oracle itself, with no kernel
    involved) moves dQ by about a tenth of its size, so end-to-end checks run
    on the unscaled workloads and the sweeps.

Tolerance, per gradient tensor over the compared elements (derived from an
emulation of the kernels' roundings -- bf16 P and dS operands, fp32 accumulation,
bf16 outputs, and for the end-to-end checks D from the bf16 O -- whose worst
cases on the workload shapes were 5.7e-3 and 9.6e-3):
    max |g - g_ref|  <= 2e-2  * max |g_ref|  + 1e-4
    mean |g - g_ref| <= 2.5e-2 * mean |g_ref| + 1e-5
The absolute floors cover gradients that are exactly zero in the definition
(one key, fully masked rows), where the kernel carries fp32 rounding noise.
"""
import numpy as np
import pytest

import oracle
from flashattention_forward_attn_amd import binding, inputs
from tests.gpu_helpers import cuda, oracle_threads, to_device

pytestmark = pytest.mark.gpu

MAX_REL, MAX_FLOOR = 2e-2, 1e-4
MEAN_REL, MEAN_FLOOR = 2.5e-2, 1e-5


def check(name, g, ref, what):
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), f"{what} {name}: non-finite gradient"
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    bound_max = MAX_REL * float(np.abs(ref).max(initial=0.0)) + MAX_FLOOR
    bound_mean = MEAN_REL * float(np.abs(ref).mean()) + MEAN_FLOOR
    assert mx <= bound_max, f"{what} {name}: max err {mx:.3g} > {bound_max:.3g}"
    assert mean <= bound_mean, f"{what} {name}: mean err {mean:.3g} > {bound_mean:.3g}"
    return mx, mean


def stored(o, lse):
    """The oracle's O and LSE rounded to the storage types the backward consumes:
    (bf16 O as float64, fp32 LSE as float64)."""
    import torch
    o16 = torch.from_numpy(np.ascontiguousarray(o, np.float64)).to(torch.bfloat16)
    return o16.double().numpy(), np.asarray(lse, np.float32).astype(np.float64)


def run_backward(x, g, kv_limit=None, given=None):
    """HIP backward on x's inputs and dO g; float64 numpy gradients.

    The O and LSE it consumes come from the HIP forward, except that `given`
    = (b, h, o_head, lse_head) replaces head (b, h) of both (values exactly
    representable in the storage types), or `given` = (o, lse) replaces all."""
    torch = cuda()
    q, k, v, lim = to_device(x)
    if kv_limit is not None:
        lim = torch.from_numpy(np.ascontiguousarray(kv_limit, np.int32)).cuda()
    w = x.workload
    o, lse = binding.attention(q, k, v, causal=w.causal, scale=w.scale, kv_limit=lim)
    if given is not None and len(given) == 2:
        o.copy_(torch.from_numpy(given[0]).to(torch.bfloat16))
        lse.copy_(torch.from_numpy(given[1]).float())
    elif given is not None:
        b, h, o_head, lse_head = given
        o[b, h].copy_(torch.from_numpy(o_head).to(torch.bfloat16))
        lse[b, h].copy_(torch.from_numpy(lse_head).float())
    dout = torch.from_numpy(g.dout_bits.view(np.int16)).view(torch.bfloat16).cuda()
    dq, dk, dv = binding.attention_backward(q, k, v, o, lse, dout, causal=w.causal, scale=w.scale, kv_limit=lim)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(dq), f(dk), f(dv)


SWEEP_N = [1, 5, 17, 64, 65, 130, 200, 257]


@pytest.mark.parametrize("mask", ["none", "some_zero", "out_of_range"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SWEEP_N)
def test_backward_sweep(N, causal, d, mask):
    w = inputs.custom(f"bwd_n{N}", "bf16", 2, 2, N, d, causal, seed=N + 7 * d)
    x = inputs.generate(w)
    g = inputs.grad_output(w)
    lim = None if mask == "none" else inputs.random_kv_limit(w.B, w.N, seed=N + 3, kind=mask)
    got = run_backward(x, g, kv_limit=lim)
    ref = oracle.attention_bwd(x.q, x.k, x.v, g.dout, causal=causal, scale=w.scale, kv_limit=lim,
                               nthreads=oracle_threads())
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        check(name, a, b, f"N={N} causal={causal} d={d} mask={mask}")


@pytest.mark.parametrize("mask", ["none", "some_zero", "key_padding"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 130, 257])
def test_backward_given_output_sweep(N, causal, d, mask):
    """The backward alone, fed the oracle's stored O and LSE, on sharp rows (scores
    scaled by 8, uniform V) where the rounding of O matters most."""
    w = inputs.custom(f"bwd_sharp_n{N}", "bf16", 2, 2, N, d, causal, seed=N + 11 * d, qk_mult=8.0,
                      v_dist="uniform", key_padding=(mask == "key_padding"))
    x = inputs.generate(w)
    g = inputs.grad_output(w)
    lim = x.kv_limit if mask != "some_zero" else inputs.random_kv_limit(w.B, w.N, seed=N + 5, kind=mask)
    o, lse = oracle.attention(x.q, x.k, x.v, causal=causal, scale=w.scale, kv_limit=lim, nthreads=oracle_threads())
    o_st, lse_st = stored(o, lse)
    got = run_backward(x, g, kv_limit=lim, given=(o_st, lse_st))
    ref = oracle.attention_bwd(x.q, x.k, x.v, g.dout, causal=causal, scale=w.scale, kv_limit=lim,
                               nthreads=oracle_threads(), o=o_st)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        check(name, a, b, f"N={N} causal={causal} d={d} mask={mask}")


WORKLOAD_NAMES = ["bf16_b4h16n2048d64", "bf16_causal_b2h32n4096d128", "bf16_causal_b1h16n16384d128",
                  "bf16_keypad_b8h32n1024d128"]


def checked_head(x):
    """(b, h): the head of a workload whose every row is checked (for key padding,
    the batch item with the fully masked query block)."""
    w = x.workload
    rng = np.random.default_rng(5)
    b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
    if x.masked_batch is not None:
        b = x.masked_batch
    return b, h


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_backward_workload_whole_head(name):
    """Full-size workloads, the backward alone: every gradient computed on the GPU
    with head (b, h)'s O and LSE taken from the oracle; every row of that head's
    dQ, dK and dV checked against the oracle given the same O."""
    w = inputs.WORKLOADS[name]
    x = inputs.generate(w)
    g = inputs.grad_output(w)
    b, h = checked_head(x)
    rows = np.arange(w.N)
    ids = (b * w.H + h) * w.N + rows
    o_head, lse_head = oracle.attention_rows(x.q, x.k, x.v, ids, causal=w.causal, scale=w.scale,
                                             kv_limit=x.kv_limit, nthreads=oracle_threads())
    o_st, lse_st = stored(o_head, lse_head)
    dq, dk, dv = run_backward(x, g, given=(b, h, o_st, lse_st))
    rq, rk, rv = oracle.attention_bwd_sample(x.q, x.k, x.v, g.dout, b, h, rows, rows, causal=w.causal,
                                             scale=w.scale, kv_limit=x.kv_limit, nthreads=oracle_threads(),
                                             o_head=o_st)
    check("dq", dq[b, h], rq, name)
    check("dk", dk[b, h], rk, name)
    check("dv", dv[b, h], rv, name)
    for t in (dq, dk, dv):
        assert np.all(np.isfinite(t)), name


@pytest.mark.parametrize("name", [n for n in WORKLOAD_NAMES if inputs.WORKLOADS[n].qk_mult == 1.0])
def test_backward_workload_end_to_end_whole_head(name):
    """Full-size unscaled workloads, HIP forward then HIP backward, every row of
    one head against the exact gradients."""
    w = inputs.WORKLOADS[name]
    x = inputs.generate(w)
    g = inputs.grad_output(w)
    b, h = checked_head(x)
    rows = np.arange(w.N)
    dq, dk, dv = run_backward(x, g)
    rq, rk, rv = oracle.attention_bwd_sample(x.q, x.k, x.v, g.dout, b, h, rows, rows, causal=w.causal,
                                             scale=w.scale, kv_limit=x.kv_limit, nthreads=oracle_threads())
    check("dq", dq[b, h], rq, name)
    check("dk", dk[b, h], rk, name)
    check("dv", dv[b, h], rv, name)


def test_backward_deterministic():
    w = inputs.custom("bwd_det", "bf16", 1, 4, 777, 128, True, seed=3)
    x, g = inputs.generate(w), inputs.grad_output(w)
    a = run_backward(x, g)
    b = run_backward(x, g)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_backward_masked_rows_have_no_query_gradient():
    """Rows with no valid key: zero dq, and their dO reaches no key."""
    w = inputs.custom("bwd_mask", "bf16", 2, 2, 150, 64, False, seed=9)
    x, g = inputs.generate(w), inputs.grad_output(w)
    lim = inputs.random_kv_limit(w.B, w.N, seed=11, kind="some_zero")
    dq, dk, dv = run_backward(x, g, kv_limit=lim)
    dead = lim == 0
    for b in range(w.B):
        assert np.all(dq[b][:, dead[b]] == 0.0)
    # changing dO on the masked rows changes nothing
    g2 = inputs.GradOutput(g.dout.copy(), g.dout_bits.copy())
    g2.dout_bits[:, :, :, :][np.broadcast_to(dead[:, None, :, None], g2.dout_bits.shape)] = 0x3F80  # 1.0
    dq2, dk2, dv2 = run_backward(x, g2, kv_limit=lim)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
