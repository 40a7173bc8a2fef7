"""Pins for the oracle's FP8 forward: each compares it with something other than itself.

  - E4M3 encoding against the format's own table (written out here from the
    OCP definition): every representable value encodes to its code, midpoints
    between neighbours go to the even code, values just beside a midpoint go
    to the nearer neighbour;
  - the scale rule: per tile, amax <= 448 * 2^e and amax > 448 * 2^(e-1)
    (the smallest such e); an all-zero tile gets e = 0; tiles never mix heads;
  - the rotation equals scipy's Sylvester-Hadamard matrix applied to signs * x
    (to fp32 rounding) and multiplies every dot product by exactly d;
  - the dequantised values are within half an E4M3 step of the rotated ones;
  - attention on the codes equals the (separately pinned) forward oracle on
    the dequantised values, scores divided by d for rotated inputs;
  - the page's claim: with outlier features, random signs + Hadamard + one
    scale per tile give a lower RMSE against exact attention than one scale
    per tensor without rotation.
The last test plants plausible mistakes in a copy of the oracle's source.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

E4M3 = oracle.e4m3_values()
FINITE = [c for c in range(256) if not np.isnan(E4M3[c])]


def _dequant(codes, exps, tile):
    B, H, N, d = codes.shape
    rows = np.arange(N) // tile
    return E4M3[codes] * np.exp2(exps[:, :, rows].astype(np.float64))[..., None]


def pin_e4m3_encoding(lib):
    pos = sorted((E4M3[c], c) for c in FINITE if E4M3[c] > 0)
    vals = np.array([v for v, _ in pos])
    # one row per probe value; 448 sits in every tile so that e = 0
    probes, expect = [], []
    for v, c in pos:
        probes.append(v); expect.append(c)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (v0 + v1) / 2
        probes.append(mid); expect.append(c0 if c0 % 2 == 0 else c1)
        probes.append(np.nextafter(np.float32(mid), np.float32(0))); expect.append(c0)
        probes.append(np.nextafter(np.float32(mid), np.float32(1e9))); expect.append(c1)
    probes.append(2.0 ** -10); expect.append(0)            # half the smallest subnormal: tie to 0
    probes.append(1.5 * 2.0 ** -9); expect.append(2)       # tie between codes 1 and 2: even
    n = len(probes)
    x = np.zeros((1, 1, n, 2))
    x[0, 0, :, 0] = np.float32(probes)
    x[0, 0, :, 1] = 448.0
    codes, exps = oracle.fp8_quantize(x, None, tile_rows=n, lib=lib)
    assert exps.ravel().tolist() == [0]
    np.testing.assert_array_equal(codes[0, 0, :, 0], np.array(expect, np.uint8))
    # negative values mirror through the sign bit
    codes_n, _ = oracle.fp8_quantize(-x, None, tile_rows=n, lib=lib)
    np.testing.assert_array_equal(codes_n[0, 0, :, 0], np.array(expect, np.uint8) | 0x80)
    assert vals.max() == 448.0


def pin_scale_rule(lib):
    r = np.random.default_rng(3)
    x = r.standard_normal((2, 3, 150, 16)) * np.exp2(r.integers(-20, 20, size=(2, 3, 150, 1)))
    x[1, 2, 64:128] = 0.0                                  # an all-zero tile
    codes, exps = oracle.fp8_quantize(x, None, tile_rows=64, lib=lib)
    for b in range(2):
        for h in range(3):
            for t in range(3):
                tile = np.float32(x[b, h, 64 * t:64 * t + 64])
                amax = float(np.abs(tile).max())
                e = int(exps[b, h, t])
                if amax == 0.0:
                    assert e == 0
                    continue
                assert amax <= 448.0 * 2.0 ** e and amax > 448.0 * 2.0 ** (e - 1), (b, h, t, amax, e)
    # a change in one head leaves the other heads' tiles alone
    x2 = x.copy(); x2[0, 1] *= 1024.0
    _, exps2 = oracle.fp8_quantize(x2, None, tile_rows=64, lib=lib)
    np.testing.assert_array_equal(np.delete(exps2, 1, axis=1)[0], np.delete(exps, 1, axis=1)[0])
    np.testing.assert_array_equal(exps2[1], exps[1])
    np.testing.assert_array_equal(exps2[0, 1], exps[0, 1] + 10)


def pin_rotation(lib):
    r = np.random.default_rng(4)
    for d in (8, 64, 128):
        signs = r.choice([-1, 1], d).astype(np.int8)
        x = np.float32(r.standard_normal((5, d)))
        y = oracle.fp8_rotate(x, signs, lib=lib)
        ref = (scipy.linalg.hadamard(d) @ (signs * x.astype(np.float64)).T).T
        np.testing.assert_allclose(y, ref, rtol=0, atol=4e-6 * np.abs(ref).max())
        g = y.astype(np.float64) @ y.astype(np.float64).T
        np.testing.assert_allclose(g, d * (x.astype(np.float64) @ x.astype(np.float64).T), rtol=1e-5, atol=1e-4)


def pin_dequantisation_error(lib):
    r = np.random.default_rng(5)
    x = r.standard_normal((1, 2, 96, 64))
    signs = r.choice([-1, 1], 64).astype(np.int8)
    codes, exps = oracle.fp8_quantize(x, signs, tile_rows=32, lib=lib)
    y = oracle.fp8_rotate(x, signs, lib=lib).astype(np.float64)
    deq = _dequant(codes, exps, 32)
    scale = np.exp2(exps[:, :, np.arange(96) // 32].astype(np.float64))[..., None]
    mag = np.abs(y) / scale                                    # in units of the tile's scale
    step = np.where(mag >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - y) <= 0.5 * step * scale * (1 + 1e-12))


def pin_attention_on_codes(lib):
    r = np.random.default_rng(6)
    B, H, N, d = 1, 2, 70, 64
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    signs = r.choice([-1, 1], d).astype(np.int8)
    lim = r.integers(0, N + 1, size=(B, N)).astype(np.int32)
    for rotated in (False, True):
        sg = signs if rotated else None
        qc, qe = oracle.fp8_quantize(q, sg, tile_rows=32, lib=lib)
        kc, ke = oracle.fp8_quantize(k, sg, tile_rows=64, lib=lib)
        for causal in (False, True):
            o, lse = oracle.attention_fp8(qc, qe, 32, kc, ke, 64, v, causal=causal, rotated=rotated, kv_limit=lim,
                                          lib=lib)
            div = np.sqrt(d) if rotated else 1.0
            ro, rl = oracle.attention(_dequant(qc, qe, 32) / div, _dequant(kc, ke, 64) / div, v, causal=causal,
                                      kv_limit=lim, lib=lib)
            np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(rl))
            fin = np.isfinite(rl)
            np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)


def outlier_inputs(seed, B=1, H=1, N=512, d=128):
    """Normal Q and K with a few feature columns scaled up (the page's simulated outliers)."""
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((B, H, N, d)) for _ in range(3))
    cols = r.choice(d, 4, replace=False)
    q[..., cols] *= 20.0
    k[..., cols] *= 20.0
    return q * 0.25, k * 0.25, v


def fp8_rmse(q, k, v, scheme, seed=7, lib=None):
    """RMSE of O against exact attention for 'tile_rotated' or 'tensor_plain' quantisation."""
    B, H, N, d = q.shape
    ro, _ = oracle.attention(q, k, v, lib=lib)
    if scheme == "tile_rotated":
        signs = np.random.default_rng(seed).choice([-1, 1], d).astype(np.int8)
        qc, qe = oracle.fp8_quantize(q, signs, tile_rows=32, lib=lib)
        kc, ke = oracle.fp8_quantize(k, signs, tile_rows=64, lib=lib)
        o, _ = oracle.attention_fp8(qc, qe, 32, kc, ke, 64, v, rotated=True, lib=lib)
    else:
        qc, qe = oracle.fp8_quantize(q, None, tile_rows=N, lib=lib)   # one scale for the (one-head) tensor
        kc, ke = oracle.fp8_quantize(k, None, tile_rows=N, lib=lib)
        o, _ = oracle.attention_fp8(qc, qe, N, kc, ke, N, v, rotated=False, lib=lib)
    return float(np.sqrt(np.mean((o - ro) ** 2)))


def pin_incoherent_processing_lowers_rmse(lib):
    for seed in (8, 9):
        q, k, v = outlier_inputs(seed)
        ours = fp8_rmse(q, k, v, "tile_rotated", lib=lib)
        base = fp8_rmse(q, k, v, "tensor_plain", lib=lib)
        assert ours < base / 1.5, (seed, ours, base)


PINS = [pin_e4m3_encoding, pin_scale_rule, pin_rotation, pin_dequantisation_error, pin_attention_on_codes,
        pin_incoherent_processing_lowers_rmse]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle._library())


_FP8 = "static double e4m3_value("
MUTATIONS = {
    "butterfly_adds_twice": ("            y[i + h] = a - b;", "            y[i + h] = a + b;"),
    "signs_ignored": ("for (int64_t c = 0; c < d; ++c) y[c] = (float)x[c] * (float)signs[c];",
                      "for (int64_t c = 0; c < d; ++c) y[c] = (float)x[c];"),
    "exponent_not_minimal": ("int e = (m <= 0.875) ? k - 9 : k - 8;", "int e = (m <= 0.875) ? k - 8 : k - 7;"),
    "ties_away_from_zero": ("const double r = nearbyint(a / step);", "const double r = floor(a / step + 0.5);"),
    "score_divisor_dropped": ("scale / score_div, kv_limit, nthreads);", "scale, kv_limit, nthreads);"),
    "k_exponent_by_q_tile": ("kd[i] = ldexp(e4m3_value(kc[i]), ke[bh * nkt + r / k_tile]);",
                             "kd[i] = ldexp(e4m3_value(kc[i]), ke[bh * nkt + r / q_tile]);"),
    "subnormal_step_wrong": ("if (E2 < -6) return sign | (uint8_t)(int)(v / ldexp(1.0, -9));",
                             "if (E2 < -6) return sign | (uint8_t)(int)(v / ldexp(1.0, -8));"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    start = src.index(_FP8)
    assert old in src[start:], f"mutation {name!r} no longer matches the oracle source"
    path = tmp_path / "fa_oracle_mut.c"
    path.write_text(src[:start] + src[start:].replace(old, new, 1))
    lib = oracle.load(oracle.compile_library(str(path), str(tmp_path / "libfa_oracle_mut.so")))
    failures = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError):
            failures.append(pin.__name__)
    assert failures, f"planted mistake {name!r} passed every pin"
