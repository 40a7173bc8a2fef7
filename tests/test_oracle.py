"""Pins for the fp64 oracle: each check compares it with something other than itself.

Kinds of pin used (every function of the oracle is covered by several):
  - values the pages print for worked examples (tests/golden/*.json);
  - a library routine the definition reduces to (scipy's softmax and logsumexp
    when V is the identity, so O is the attention matrix itself);
  - brute force on tiny inputs in pure Python with math.fsum and no max
    subtraction, at positive, negative and zero scale;
  - closed forms (Q = 0 or scale = 0, N = 1, the causal first row, constant V,
    shifted scores);
  - invariants (keys and values permuted together; splitting rows into blocks,
    against the test-side online recurrence in online_reference.py);
  - large-magnitude logits, where a missing max subtraction overflows.
The last test plants plausible mistakes in a copy of the oracle's source and
checks that every one of them fails at least one pin.
"""
import json
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from tests.online_reference import mask_matrix, online_attention

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _one_query(scores, values, kv_limit=None, lib=None):
    """One query row of width 1: q = 1, keys = the scores, scale 1."""
    n = len(scores)
    q = np.ones((1, 1, n, 1))
    k = np.asarray(scores, np.float64).reshape(1, 1, n, 1)
    v = np.asarray(values, np.float64).reshape(1, 1, n, 1)
    lim = None
    if kv_limit is not None:
        lim = np.full((1, n), kv_limit, np.int32)
    o, lse = oracle.attention(q, k, v, causal=False, scale=1.0, kv_limit=lim, lib=lib)
    return o[0, 0, 0, 0], lse[0, 0, 0]


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


# --------------------------------------------------------------------------- pins
# Each pin takes the library handle so the mutation test can run it against a
# deliberately broken build.

def pin_worked_example(lib, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "online_softmax_worked_example.json")))
    names = {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0)}
    scores = [names[s] for s in g["scores"]]
    o, lse = _one_query(scores, g["values"], lib=lib)
    assert abs(o - 17.0 / 6.0) < 1e-14, o
    assert abs(lse - math.log(6.0)) < 1e-14
    # the first block alone (keys 0 and 1) is the prefix the page stops at:
    # m = ln 2, l = 1.5, u = 2.5, so O = u / l and LSE = m + ln l
    first = g["after_first_block"]
    o2, lse2 = _one_query(scores, g["values"], kv_limit=2, lib=lib)
    assert abs(o2 - first["u"] / first["l"]) < 1e-14
    assert abs(lse2 - (names[first["m"]] + math.log(first["l"]))) < 1e-14
    second = g["after_second_block"]
    assert abs(o - 17.0 / 3.0 / second["l"]) < 1e-14


def pin_six_scores(lib, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "online_softmax_six_scores.json")))
    scores = [s for blk in g["blocks"] for s in blk]
    values = [0.0] * len(scores)
    seen = 0
    for blk, m, l2 in zip(g["blocks"], g["m_after_block"], g["l_after_block_2dp"]):
        seen += len(blk)
        _, lse = _one_query(scores, values, kv_limit=seen, lib=lib)
        # LSE of the prefix is m + ln l; the page prints l to two decimals
        assert round(math.exp(lse - m), 2) == l2, (seen, math.exp(lse - m), l2)
        assert max(scores[:seen]) == m


def pin_softmax_library(lib, golden_dir=None):
    """V = I makes O the attention matrix: compare with scipy's softmax."""
    B, H, N = 2, 3, 12
    q = _rand((B, H, N, N), 1)
    k = _rand((B, H, N, N), 2)
    v = np.broadcast_to(np.eye(N), (B, H, N, N)).copy()
    lim = np.random.default_rng(3).integers(0, N + 1, size=(B, N)).astype(np.int32)
    scale = 0.37
    for causal in (False, True):
        for kv in (None, lim):
            o, lse = oracle.attention(q, k, v, causal=causal, scale=scale, kv_limit=kv, lib=lib)
            for b in range(B):
                ok = mask_matrix(N, causal, None if kv is None else kv[b])
                for h in range(H):
                    s = scale * (q[b, h] @ k[b, h].T)
                    s = np.where(ok, s, -np.inf)
                    full = ok.any(axis=1)
                    ref = np.zeros((N, N))
                    ref[full] = scipy.special.softmax(s[full], axis=1)
                    ref_lse = np.full(N, -np.inf)
                    ref_lse[full] = scipy.special.logsumexp(s[full], axis=1)
                    np.testing.assert_allclose(o[b, h], ref, rtol=0, atol=1e-14)
                    np.testing.assert_allclose(lse[b, h][full], ref_lse[full], rtol=1e-14, atol=1e-14)
                    assert np.all(np.isneginf(lse[b, h][~full]))
                    # rows of a softmax sum to one; masked entries are exactly zero
                    np.testing.assert_allclose(o[b, h][full].sum(axis=1), 1.0, atol=1e-14)
                    assert np.all(o[b, h][~ok] == 0.0)


def _brute(q, k, v, causal, scale, lim):
    """Pure-Python attention, direct sum exp(s) v / sum exp(s), no max subtraction."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N)
                        if (not causal or j <= i) and (lim is None or j < lim[b, i])]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                w = [math.exp(scale * math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)))
                     for j in keys]
                den = math.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(wj * v[b, h, j, c] for wj, j in zip(w, keys)) / den
                lse[b, h, i] = math.log(den)
    return o, lse


def pin_brute_force(lib, golden_dir=None):
    for seed, (B, H, N, d) in enumerate([(1, 1, 1, 1), (1, 2, 2, 3), (2, 1, 3, 2), (2, 2, 4, 3)]):
        q, k, v = _rand((B, H, N, d), 10 + seed), _rand((B, H, N, d), 20 + seed), _rand((B, H, N, d), 30 + seed)
        lim = np.random.default_rng(40 + seed).integers(0, N + 1, size=(B, N)).astype(np.int32)
        for causal, kv, scale in itertools.product((False, True), (None, lim), (0.8, -0.8, 0.0)):
            o, lse = oracle.attention(q, k, v, causal=causal, scale=scale, kv_limit=kv, lib=lib)
            ro, rl = _brute(q, k, v, causal, scale, kv)
            np.testing.assert_allclose(o, ro, rtol=1e-13, atol=1e-14)
            fin = np.isfinite(rl)
            np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-13, atol=1e-14)
            assert np.array_equal(np.isneginf(lse), ~fin)


def pin_closed_forms(lib, golden_dir=None):
    B, H, N, d = 2, 2, 9, 4
    k, v = _rand((B, H, N, d), 50), _rand((B, H, N, d), 51)
    lim = np.array([[9, 3, 0, 5, 9, 1, 2, 7, 4], [0] * 9], np.int32)
    # Q = 0: uniform weights over the valid keys
    o, lse = oracle.attention(np.zeros((B, H, N, d)), k, v, causal=True, scale=1.0, kv_limit=lim, lib=lib)
    for b in range(B):
        ok = mask_matrix(N, True, lim[b])
        for i in range(N):
            n = ok[i].sum()
            if n == 0:
                assert np.all(o[b, :, i] == 0) and np.all(np.isneginf(lse[b, :, i]))
            else:
                np.testing.assert_allclose(o[b, :, i], v[b][:, ok[i]].mean(axis=1), atol=1e-14)
                np.testing.assert_allclose(lse[b, :, i], math.log(n), atol=1e-14)
    # scale = 0 (any Q): uniform weights as well
    o0, l0 = oracle.attention(_rand((B, H, N, d), 58, 5.0), k, v, causal=True, scale=0.0, kv_limit=lim, lib=lib)
    np.testing.assert_allclose(o0, o, atol=1e-14)
    np.testing.assert_array_equal(np.isneginf(l0), np.isneginf(lse))
    np.testing.assert_allclose(l0[np.isfinite(l0)], lse[np.isfinite(lse)], atol=1e-14)
    # N = 1: the only key's value; LSE is its score
    q1, k1, v1 = _rand((1, 3, 1, 5), 52), _rand((1, 3, 1, 5), 53), _rand((1, 3, 1, 5), 54)
    o, lse = oracle.attention(q1, k1, v1, scale=0.5, lib=lib)
    np.testing.assert_array_equal(o, v1)
    np.testing.assert_allclose(lse[0, :, 0], 0.5 * (q1[0, :, 0] * k1[0, :, 0]).sum(-1), rtol=1e-15)
    # causal row 0 sees only key 0
    q2 = _rand((B, H, N, d), 55)
    o, lse = oracle.attention(q2, k, v, causal=True, scale=0.3, lib=lib)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * (q2[:, :, 0] * k[:, :, 0]).sum(-1), rtol=1e-15)
    # constant V gives that constant
    o, _ = oracle.attention(q2, k, np.full((B, H, N, d), -1.75), causal=False, scale=0.3, lib=lib)
    np.testing.assert_allclose(o, -1.75, rtol=1e-15)
    # shift invariance: one extra dimension with q = t_i and k = 1 adds scale*t_i to row i
    t = _rand((B, H, N, 1), 56)
    qx = np.concatenate([q2, t], axis=-1)
    kx = np.concatenate([k, np.ones((B, H, N, 1))], axis=-1)
    vx = np.concatenate([v, _rand((B, H, N, 1), 57)], axis=-1)
    o0, l0 = oracle.attention(q2, k, v, causal=True, scale=0.3, lib=lib)
    o1, l1 = oracle.attention(qx, kx, vx, causal=True, scale=0.3, lib=lib)
    np.testing.assert_allclose(o1[..., :d], o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + 0.3 * t[..., 0], atol=1e-12)


def pin_permutation(lib, golden_dir=None):
    B, H, N, d = 2, 3, 33, 8
    q, k, v = _rand((B, H, N, d), 60), _rand((B, H, N, d), 61), _rand((B, H, N, d), 62)
    perm = np.random.default_rng(63).permutation(N)
    o0, l0 = oracle.attention(q, k, v, scale=0.4, lib=lib)
    o1, l1 = oracle.attention(q, k[:, :, perm], v[:, :, perm], scale=0.4, lib=lib)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, atol=1e-13)
    # permuting queries permutes the output rows
    o2, l2 = oracle.attention(q[:, :, perm], k, v, scale=0.4, lib=lib)
    np.testing.assert_allclose(o2, o0[:, :, perm], atol=1e-13)


def pin_block_split(lib, golden_dir=None):
    B, H, N, d = 2, 2, 70, 16
    q, k, v = _rand((B, H, N, d), 70, 3.0), _rand((B, H, N, d), 71, 3.0), _rand((B, H, N, d), 72)
    lim = np.random.default_rng(73).integers(0, N + 1, size=(B, N)).astype(np.int32)
    lim[0, 5:12] = 0
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal=causal, scale=0.25, kv_limit=lim, lib=lib)
        for bq, bk, thr in [(1, 1, 0.0), (7, 7, 0.0), (64, 64, 0.0), (N, N, 0.0), (16, 7, 8 * math.log(2))]:
            ro, rl = online_attention(q, k, v, causal, 0.25, lim, bq, bk, thr)
            np.testing.assert_allclose(o, ro, atol=1e-12)
            fin = np.isfinite(rl)
            np.testing.assert_allclose(lse[fin], rl[fin], atol=1e-12)
            assert np.array_equal(np.isfinite(lse), fin)


def pin_large_logits(lib, golden_dir=None):
    """Scores beyond exp's fp64 range (the key-padding workload scales Q and K by 8;
    this goes further, so that a missing max subtraction overflows)."""
    B, H, N, d = 1, 2, 20, 32
    q, k, v = _rand((B, H, N, d), 80, 20.0), _rand((B, H, N, d), 81, 20.0), _rand((B, H, N, d), 82)
    for sc in (1 / math.sqrt(d), -1 / math.sqrt(d)):
        _large_logits_case(lib, q, k, v, sc)


def _large_logits_case(lib, q, k, v, sc):
    B, H, N, d = q.shape
    o, lse = oracle.attention(q, k, v, causal=True, scale=sc, lib=lib)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for h in range(H):
        s = (q[0, h] @ k[0, h].T) * sc
        assert s.max() > 710
        for i in range(N):
            row = s[i, :i + 1]
            m = row.max()
            w = [math.exp(x - m) for x in row]
            den = math.fsum(w)
            ref = [math.fsum(w[j] * v[0, h, j, c] for j in range(i + 1)) / den for c in range(d)]
            np.testing.assert_allclose(o[0, h, i], ref, atol=1e-13)
            assert abs(lse[0, h, i] - (m + math.log(den))) < 1e-12


def pin_rows_entry(lib, golden_dir=None):
    B, H, N, d = 2, 3, 40, 8
    q, k, v = _rand((B, H, N, d), 90), _rand((B, H, N, d), 91), _rand((B, H, N, d), 92)
    lim = np.random.default_rng(93).integers(0, N + 1, size=(B, N)).astype(np.int32)
    o, lse = oracle.attention(q, k, v, causal=True, scale=0.5, kv_limit=lim, lib=lib)
    ids = np.array([0, 7, N - 1, N, 2 * N + 5, B * H * N - 1], np.int64)
    ro, rl = oracle.attention_rows(q, k, v, ids, causal=True, scale=0.5, kv_limit=lim, lib=lib)
    np.testing.assert_array_equal(ro, o.reshape(-1, d)[ids])
    np.testing.assert_array_equal(rl, lse.reshape(-1)[ids])


PINS = [pin_worked_example, pin_six_scores, pin_softmax_library, pin_brute_force, pin_closed_forms,
        pin_permutation, pin_block_split, pin_large_logits, pin_rows_entry]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, golden_dir):
    pin(oracle._library(), golden_dir)


def test_online_reference_reproduces_the_worked_example(golden_dir):
    """The test-side recurrence, split 2 + 1, passes through the page's intermediate values."""
    g = json.load(open(os.path.join(golden_dir, "online_softmax_worked_example.json")))
    s = np.array([0.0, math.log(2), math.log(3)])
    q = np.ones((1, 1, 1, 1))
    k = s.reshape(1, 1, 3, 1)
    v = np.array(g["values"]).reshape(1, 1, 3, 1)
    # run the first block only, then both blocks
    o1, l1 = online_attention(q, k[:, :, :2], v[:, :, :2], scale=1.0, block_k=2)
    first = g["after_first_block"]
    assert abs(math.exp(l1[0, 0, 0] - math.log(2)) - first["l"]) < 1e-15
    assert abs(o1[0, 0, 0, 0] * first["l"] - first["u"]) < 1e-15
    # full row in one query position: pad to a common N so both blocks are visible
    qq = np.ones((1, 1, 3, 1))
    o, lse = online_attention(qq, k, v, scale=1.0, block_k=2)
    assert abs(o[0, 0, 0, 0] - 17 / 6) < 1e-15
    assert abs(math.exp(lse[0, 0, 0] - math.log(3)) - g["after_second_block"]["l"]) < 1e-15


# Plausible mistakes, each planted into a temporary copy of the oracle's source.
MUTATIONS = {
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "exp_sign": ("double w = exp(s[j] - m);", "double w = exp(m - s[j]);"),
    "operands_transposed": ("acc += qi[c] * kh[j * d + c];",
                            "acc += q[((b * H + h) * N + j) * d + c] * k[((b * H + h) * N + i) * d + c];"),
    "causal_drops_diagonal": ("if (causal && j > i) return 0;", "if (causal && j >= i) return 0;"),
    "causal_wrong_triangle": ("if (causal && j > i) return 0;", "if (causal && j < i) return 0;"),
    "limit_off_by_one": ("return j < limit;", "return j <= limit;"),
    "lse_without_max": ("*lse_row = m + log(l);", "*lse_row = log(l);"),
    "no_max_subtraction": ("double w = exp(s[j] - m);", "double w = exp(s[j]);"),
    "value_row_index": ("o_row[c] += w * vh[j * d + c];", "o_row[c] += w * vh[i * d + c];"),
    "unnormalised": ("for (int64_t c = 0; c < d; ++c) o_row[c] /= l;", ""),
    "query_head_reversed": ("const double *qi = q + ((b * H + h) * N + i) * d;",
                            "const double *qi = q + ((b * H + (H - 1 - h)) * N + i) * d;"),
    "masked_keys_in_denominator": ("if (!key_is_valid(j, i, causal, limit)) continue;\n        double w",
                                   "if (!key_is_valid(j, i, causal, limit)) { l += exp(s[j] - m); continue; }\n        double w"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, golden_dir, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation {name!r} no longer matches the oracle source"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "fa_oracle_mut.c"
    path.write_text(mutated)
    lib_path = oracle.compile_library(str(path), str(tmp_path / "libfa_oracle_mut.so"))
    lib = oracle.load(lib_path)
    failures = []
    for pin in PINS:
        try:
            pin(lib, golden_dir)
        except AssertionError as exc:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"
