"""Pins for the oracle's paged decode: each compares it with something other than itself.

  - reduction to the contiguous case: gathering each sequence's pages through
    its block table into contiguous K/V and putting the query at row 0 of a
    forward problem with key limit = the sequence length must give the
    (separately pinned) forward oracle's row 0;
  - invariance: permuting the physical pages of the pool, with the block table
    remapped accordingly, changes nothing (bit for bit);
  - closed forms: an empty sequence gives o = 0 and lse = -inf; one key gives
    o = v_0 and lse = scale <q, k_0>; q = 0 gives the mean of the sequence's
    value rows and lse = ln(len);
  - brute force: pure Python sums (math.fsum) on tiny caches, page size 1 and 3.
The last test plants plausible mistakes in a copy of the oracle's source and
checks that each fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle


def _cache(seed, B=3, H=2, d=8, page_size=4, max_pages=5, extra_pages=3, lens=None):
    """Random paged cache: distinct physical pages per sequence, shuffled in the pool."""
    r = np.random.default_rng(seed)
    if lens is None:
        lens = r.integers(0, max_pages * page_size + 1, size=B)
    lens = np.asarray(lens, np.int32)
    need = [int(-(-int(n) // page_size)) for n in lens]
    num_pages = sum(need) + extra_pages
    perm = r.permutation(num_pages)
    bt = np.zeros((B, max_pages), np.int32)
    at = 0
    for b in range(B):
        bt[b, :need[b]] = perm[at:at + need[b]]
        at += need[b]
        # unused entries point at arbitrary (valid) pages; they must be ignored
        bt[b, need[b]:] = r.integers(0, num_pages, size=max_pages - need[b])
    q = r.standard_normal((B, H, d))
    k = r.standard_normal((num_pages, H, page_size, d))
    v = r.standard_normal((num_pages, H, page_size, d))
    return q, k, v, bt, lens


def _gather(cache, bt, lens, b, page_size):
    """Keys 0..len-1 of sequence b, contiguous: (H, len, d)."""
    j = np.arange(int(lens[b]))
    return cache[bt[b, j // page_size], :, j % page_size, :].transpose(1, 0, 2)


def pin_decode_contiguous(lib):
    for seed, ps in ((1, 4), (2, 16), (3, 1)):
        q, k, v, bt, lens = _cache(seed, page_size=ps, max_pages=6 if ps > 1 else 40)
        B, H, d = q.shape
        scale = 0.37
        o, lse = oracle.decode_paged(q, k, v, bt, lens, scale=scale, lib=lib)
        N = max(1, int(lens.max()))
        for b in range(B):
            Q = np.zeros((1, H, N, d)); Q[0, :, 0, :] = q[b]
            K = np.zeros((1, H, N, d)); V = np.zeros((1, H, N, d))
            n = int(lens[b])
            K[0, :, :n] = _gather(k, bt, lens, b, ps)
            V[0, :, :n] = _gather(v, bt, lens, b, ps)
            lim = np.zeros((1, N), np.int32); lim[0, 0] = n
            ro, rl = oracle.attention(Q, K, V, scale=scale, kv_limit=lim, lib=lib)
            np.testing.assert_allclose(o[b], ro[0, :, 0], rtol=1e-12, atol=1e-13)
            if n == 0:
                assert np.all(np.isneginf(lse[b]))
            else:
                np.testing.assert_allclose(lse[b], rl[0, :, 0], rtol=1e-12, atol=1e-13)


def pin_decode_page_permutation(lib):
    q, k, v, bt, lens = _cache(11, B=4, H=3, page_size=4, max_pages=6)
    o, lse = oracle.decode_paged(q, k, v, bt, lens, lib=lib)
    perm = np.random.default_rng(12).permutation(k.shape[0])   # new position of each page
    k2 = np.empty_like(k); v2 = np.empty_like(v)
    k2[perm] = k; v2[perm] = v
    o2, lse2 = oracle.decode_paged(q, k2, v2, perm[bt].astype(np.int32), lens, lib=lib)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def pin_decode_closed_forms(lib):
    q, k, v, bt, lens = _cache(21, B=3, H=2, d=8, page_size=4, max_pages=4, lens=[0, 1, 13])
    scale = 0.5
    o, lse = oracle.decode_paged(q, k, v, bt, lens, scale=scale, lib=lib)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    np.testing.assert_allclose(o[1], v[bt[1, 0], :, 0, :], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[1], scale * np.einsum("hd,hd->h", q[1], k[bt[1, 0], :, 0, :]), rtol=1e-14)
    o0, lse0 = oracle.decode_paged(np.zeros_like(q), k, v, bt, lens, scale=scale, lib=lib)
    np.testing.assert_allclose(o0[2], _gather(v, bt, lens, 2, 4).mean(axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse0[2], math.log(13), rtol=1e-14)


def pin_decode_brute_force(lib):
    for ps in (1, 3):
        q, k, v, bt, lens = _cache(31 + ps, B=2, H=2, d=3, page_size=ps, max_pages=7 // ps + 1, lens=[5, 7])
        scale = 0.9
        o, lse = oracle.decode_paged(q, k, v, bt, lens, scale=scale, lib=lib)
        for b in range(2):
            for h in range(2):
                keys = [(int(bt[b, j // ps]), j % ps) for j in range(int(lens[b]))]
                s = [scale * math.fsum(q[b, h, c] * k[p, h, t, c] for c in range(3)) for p, t in keys]
                w = [math.exp(x) for x in s]
                tot = math.fsum(w)
                for c in range(3):
                    ref = math.fsum(wi * v[p, h, t, c] for wi, (p, t) in zip(w, keys)) / tot
                    assert abs(o[b, h, c] - ref) <= 1e-13 * (1 + abs(ref))
                assert abs(lse[b, h] - math.log(tot)) <= 1e-13 * (1 + abs(lse[b, h]))


def pin_decode_rejects_bad_cache(lib):
    q, k, v, bt, lens = _cache(41, B=2, page_size=4, max_pages=3, lens=[5, 12])
    with pytest.raises(RuntimeError):
        oracle.decode_paged(q, k, v, bt, np.array([5, 13], np.int32), lib=lib)   # longer than the table
    bad = bt.copy(); bad[1, 2] = k.shape[0]
    with pytest.raises(RuntimeError):
        oracle.decode_paged(q, k, v, bad, lens, lib=lib)                          # page outside the pool


PINS = [pin_decode_contiguous, pin_decode_page_permutation, pin_decode_closed_forms, pin_decode_brute_force,
        pin_decode_rejects_bad_cache]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle._library())


# Plausible mistakes, each planted into a temporary copy of the oracle's source
# (first occurrence inside the decode function); every one keeps all accesses
# in bounds.
_DEC = "int fa_oracle_decode_paged("
MUTATIONS = {
    "scale_dropped": ("s[j] = scale * acc;\n                    if (s[j] > m)", "s[j] = acc;\n                    if (s[j] > m)"),
    "slot_shifted": ("const double *kj = k_cache + ((page * H + h) * page_size + j % page_size) * d;",
                     "const double *kj = k_cache + ((page * H + h) * page_size + (j + 1) % page_size) * d;"),
    "value_from_wrong_head": ("const double *vj = v_cache + ((page * H + h) * page_size + j % page_size) * d;",
                              "const double *vj = v_cache + ((page * H + (h + 1) % H) * page_size + j % page_size) * d;"),
    "values_unweighted": ("for (int64_t c = 0; c < d; ++c) ov[c] += w * vj[c];",
                          "for (int64_t c = 0; c < d; ++c) ov[c] += vj[c];"),
    "lse_without_max": ("lse[bh] = m + log(l);", "lse[bh] = log(l);"),
    "not_normalised": ("for (int64_t c = 0; c < d; ++c) ov[c] /= l;\n                lse[bh]",
                       "for (int64_t c = 0; c < d; ++c) ov[c] /= 1.0;\n                lse[bh]"),
    "last_key_dropped": ("for (int64_t j = 0; j < len; ++j) {\n                    const int64_t page = block_table[b * max_pages + j / page_size];\n                    const double *vj",
                         "for (int64_t j = 0; j + 1 < len; ++j) {\n                    const int64_t page = block_table[b * max_pages + j / page_size];\n                    const double *vj"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    start = src.index(_DEC)
    assert old in src[start:], f"mutation {name!r} no longer matches the oracle source"
    mutated = src[:start] + src[start:].replace(old, new, 1)
    path = tmp_path / "fa_oracle_mut.c"
    path.write_text(mutated)
    lib = oracle.load(oracle.compile_library(str(path), str(tmp_path / "libfa_oracle_mut.so")))
    failures = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"
