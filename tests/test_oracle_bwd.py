"""Pins for the oracle's backward pass: each compares it with something other than itself.

  - central finite differences of the (separately pinned) forward oracle: the
    gradient of sum(dO * O) with respect to every entry of Q, K and V, on small
    problems with and without causal masking, key limits and a fully masked row;
  - exact invariants of the softmax Jacobian: for every row the score gradients
    sum to zero, so the key gradients of a head sum to zero, and the value
    gradients of a head sum to the output gradients of the rows that see a key;
  - closed forms: one key (P = 1: dV = dO, dQ = dK = 0) and equal keys (P uniform
    over the valid keys: dQ = 0 and dV_j = sum of dO_i / n_i over the rows i that
    see key j);
  - the row term taken from a given output O: with the exact O it equals the
    definition (sum_j P_ij dP_ij = <dO_i, O_i> because O_i = sum_j P_ij V_j);
    with O perturbed, dV is unchanged and dQ, dK move by the closed-form
    correction -scale * dD_i * P_ij applied to K_j and Q_i;
  - the sampled entry point against the full one, with and without a given O.
The last test plants plausible mistakes in a copy of the oracle's source and
checks that each one fails at least one pin.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _problem(seed, B=1, H=2, N=6, d=4, mult=1.0):
    r = np.random.default_rng(seed)
    q, k, v, g = (r.standard_normal((B, H, N, d)) * m for m in (mult, mult, 1.0, 1.0))
    return q, k, v, g


def _limits(B, N, seed):
    r = np.random.default_rng(seed)
    lim = r.integers(1, N + 1, size=(B, N)).astype(np.int32)
    lim[0, N // 2] = 0  # one fully masked row
    return lim


def _valid(N, causal, lim_row=None):
    """[N, N] validity for one batch item: row i, key j."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    ok = np.ones((N, N), bool)
    if causal:
        ok &= j <= i
    if lim_row is not None:
        ok &= j < lim_row[:, None]
    return ok


# --------------------------------------------------------------------------- pins

def pin_bwd_finite_difference(lib):
    cases = [dict(causal=False, kv=False, scale=None), dict(causal=True, kv=False, scale=0.7),
             dict(causal=False, kv=True, scale=None), dict(causal=True, kv=True, scale=1.3)]
    h = 1e-6
    for n, case in enumerate(cases):
        q, k, v, g = _problem(10 + n)
        B, H, N, d = q.shape
        lim = _limits(B, N, 20 + n) if case["kv"] else None
        kw = dict(causal=case["causal"], scale=case["scale"], kv_limit=lim, lib=lib)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, **kw)

        def loss(qq, kk, vv):
            o, _ = oracle.attention(qq, kk, vv, **kw)
            return float(np.sum(o * g))

        for which, grad in (("q", dq), ("k", dk), ("v", dv)):
            num = np.zeros_like(grad)
            for idx in np.ndindex(*grad.shape):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[which][idx] += h
                up = loss(args["q"], args["k"], args["v"])
                args[which][idx] -= 2 * h
                dn = loss(args["q"], args["k"], args["v"])
                num[idx] = (up - dn) / (2 * h)
            err = np.abs(num - grad).max()
            assert err <= 1e-6 * (1.0 + np.abs(grad).max()), (case, which, err)


def pin_bwd_invariants(lib):
    for causal in (False, True):
        for kv in (False, True):
            q, k, v, g = _problem(31, B=2, H=2, N=40, d=8)
            B, H, N, d = q.shape
            lim = _limits(B, N, 32) if kv else None
            dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal=causal, kv_limit=lim, lib=lib)
            assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
            # score gradients of each row sum to zero -> key gradients of a head sum to zero
            np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12 * (1 + np.abs(dk).max()) * N)
            # probabilities of each row with a valid key sum to one
            for b in range(B):
                valid = _valid(N, causal, None if lim is None else lim[b])
                seen = valid.any(axis=1)
                expect = g[b][:, seen].sum(axis=1)
                np.testing.assert_allclose(dv[b].sum(axis=1), expect, rtol=1e-12, atol=1e-12 * N)
                # a row that sees no key has no query gradient
                np.testing.assert_array_equal(dq[b][:, ~seen], 0.0)


def pin_bwd_closed_forms(lib):
    # one key: P = 1, so O = V and dV = dO, dQ = dK = 0
    q, k, v, g = _problem(41, N=1)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, lib=lib)
    np.testing.assert_allclose(dv, g, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    # equal keys: P uniform over each row's valid keys
    for causal in (False, True):
        q, k, v, g = _problem(42, B=1, H=1, N=9, d=3)
        k[:] = k[:, :, :1, :]
        lim = _limits(1, 9, 43)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal=causal, kv_limit=lim, lib=lib)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        valid = _valid(9, causal, lim[0]).astype(np.float64)
        n = valid.sum(axis=1)
        w = np.divide(valid, n[:, None], out=np.zeros_like(valid), where=n[:, None] > 0)  # P[i, j]
        expect = w.T @ g[0, 0]
        np.testing.assert_allclose(dv[0, 0], expect, rtol=1e-13, atol=1e-14)


def _probabilities(q, k, lse, causal, scale, lim):
    """P[b, h, i, j] from the forward oracle's lse (0 off the valid keys)."""
    B, H, N, d = q.shape
    P = np.zeros((B, H, N, N))
    for b in range(B):
        valid = _valid(N, causal, None if lim is None else lim[b])
        for h in range(H):
            s = scale * q[b, h] @ k[b, h].T
            L = lse[b, h][:, None]
            ok = valid & np.isfinite(L)
            P[b, h] = np.where(ok, np.exp(np.where(ok, s - np.where(np.isfinite(L), L, 0.0), -np.inf)), 0.0)
    return P


def pin_bwd_given_output(lib):
    for causal in (False, True):
        q, k, v, g = _problem(61, B=2, H=2, N=24, d=8, mult=2.0)
        B, H, N, d = q.shape
        lim = _limits(B, N, 62)
        scale = 0.6
        kw = dict(causal=causal, scale=scale, kv_limit=lim, lib=lib)
        o, lse = oracle.attention(q, k, v, **kw)
        ref = oracle.attention_bwd(q, k, v, g, **kw)
        # the exact output: the same gradients as the definition
        for a, r in zip(oracle.attention_bwd(q, k, v, g, o=o, **kw), ref):
            np.testing.assert_allclose(a, r, rtol=1e-11, atol=1e-12)
        # a perturbed output shifts D by dD_i = <dO_i, o'_i - o_i>
        r = np.random.default_rng(63)
        o2 = o + 1e-2 * r.standard_normal(o.shape)
        dq2, dk2, dv2 = oracle.attention_bwd(q, k, v, g, o=o2, **kw)
        dD = np.sum(g * (o2 - o), axis=-1)  # [B, H, N]
        P = _probabilities(q, k, lse, causal, scale, lim)
        dq_shift = -scale * dD[..., None] * (P @ k)
        dk_shift = -scale * np.swapaxes(P * dD[..., None], -1, -2) @ q
        np.testing.assert_allclose(dv2, ref[2], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dq2 - ref[0], dq_shift, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dk2 - ref[1], dk_shift, rtol=1e-9, atol=1e-12)


def pin_bwd_sample_entry(lib):
    q, k, v, g = _problem(51, B=2, H=3, N=33, d=8)
    lim = _limits(2, 33, 52)
    o_given = np.random.default_rng(53).standard_normal(q.shape)
    for causal in (False, True):
        for o in (None, o_given):
            dq, dk, dv = oracle.attention_bwd(q, k, v, g, causal=causal, kv_limit=lim, lib=lib, o=o)
            rows_q, rows_k = [0, 5, 16, 32], [1, 16, 31]
            sq, sk, sv = oracle.attention_bwd_sample(q, k, v, g, 1, 2, rows_q, rows_k, causal=causal,
                                                     kv_limit=lim, lib=lib,
                                                     o_head=None if o is None else o[1, 2])
            np.testing.assert_allclose(sq, dq[1, 2, rows_q], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(sk, dk[1, 2, rows_k], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(sv, dv[1, 2, rows_k], rtol=1e-13, atol=1e-15)


PINS = [pin_bwd_finite_difference, pin_bwd_invariants, pin_bwd_closed_forms, pin_bwd_given_output,
        pin_bwd_sample_entry]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle._library())


# Plausible mistakes in the backward pass, each planted into a temporary copy of
# the oracle's source (the first occurrence is in the full backward function or
# in the per-head row statistics it uses).
MUTATIONS = {
    "delta_term_dropped": ("const double ds = p * (dp - dd_h[i]);", "const double ds = p * dp;"),
    "delta_from_wrong_value_row": ("for (int64_t c = 0; c < d; ++c) dp += dh[i * d + c] * vh[j * d + c];",
                                   "for (int64_t c = 0; c < d; ++c) dp += dh[i * d + c] * vh[i * d + c];"),
    "dv_wrong_gradient_row": ("dvh[j * d + c] += p * dh[i * d + c];", "dvh[j * d + c] += p * dh[j * d + c];"),
    "dq_scale_dropped": ("dqh[i * d + c] += scale * ds * kh[j * d + c];", "dqh[i * d + c] += ds * kh[j * d + c];"),
    "dk_wrong_operand": ("dkh[j * d + c] += scale * ds * qh[i * d + c];",
                         "dkh[j * d + c] += scale * ds * kh[i * d + c];"),
    "p_without_lse": ("const double p = exp(scale * sij - lse_h[i]);", "const double p = exp(scale * sij);"),
    "causal_drops_diagonal_in_backward": (
        "if (!key_is_valid(j, i, causal, limit)) continue;\n                        double sij = 0.0, dp = 0.0;",
        "if (!key_is_valid(j, i, causal, limit) || (causal && j == i)) continue;\n"
        "                        double sij = 0.0, dp = 0.0;"),
    "given_output_wrong_row": ("for (int64_t c = 0; c < d; ++c) acc += dh[i * d + c] * oh[i * d + c];",
                               "for (int64_t c = 0; c < d; ++c) acc += dh[i * d + c] * oh[c];"),
    "sample_given_output_ignored": ("if (lse_h[i] != -INFINITY && !o_head) {", "if (lse_h[i] != -INFINITY) {"),
    "dp_wrong_gradient_row": ("                            dp += dh[i * d + c] * vh[j * d + c];\n                        }\n"
                              "                        const double p",
                              "                            dp += dh[j * d + c] * vh[j * d + c];\n                        }\n"
                              "                        const double p"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation {name!r} no longer matches the oracle source"
    path = tmp_path / "fa_oracle_mut.c"
    path.write_text(src.replace(old, new, 1))
    lib = oracle.load(oracle.compile_library(str(path), str(tmp_path / "libfa_oracle_mut.so")))
    failures = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"
