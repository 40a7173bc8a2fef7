"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls anything here, and this package imports
nothing from the product.

The arithmetic lives in ``fa_oracle.c`` (plain C, fp64, OpenMP over rows); this
module compiles it with gcc and calls it through ctypes.  What it computes and
which passages it follows are stated in the header of ``fa_oracle.c``:
O = softmax(scale * Q K^T + M) V and LSE = log sum exp(scale * Q K^T + M) per
row, M being 0 on valid keys and -inf elsewhere, a row with no valid key giving
O = 0 and LSE = -inf; and the backward pass, the gradients dQ, dK, dV of
sum(dO * O) for a given dO, by the chain rule through the row softmax
(optionally with the row term D_i = <dO_i, O_i> taken from a caller's stored O);
decode, one query per sequence over a paged key/value cache reached through a
block table; and the FP8 forward: Q and K rotated by random signs and a
Hadamard transform, encoded to E4M3 with one power-of-two scale per tile, then
attention on the dequantised values.

Parity: every function here is pinned, by ``tests/test_oracle.py`` (forward),
``tests/test_oracle_bwd.py`` (backward), ``tests/test_oracle_decode.py``
(paged decode) and ``tests/test_oracle_fp8.py`` (FP8), against the pages' worked
examples, closed forms, invariants, finite differences and brute force; none
is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "fa_oracle.c")
LIBRARY = os.path.join(_HERE, "libfa_oracle.so")

_lib = None


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def load(path: str = LIBRARY):
    """Load a compiled oracle library and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.fa_oracle_fwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                  ctypes.c_int, ctypes.c_double, ip, ctypes.c_int]
    lib.fa_oracle_fwd.restype = ctypes.c_int
    lib.fa_oracle_rows.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                   ctypes.c_int, ctypes.c_double, ip, i64, lp, ctypes.c_int]
    lib.fa_oracle_rows.restype = ctypes.c_int
    lib.fa_oracle_max_threads.argtypes = []
    lib.fa_oracle_max_threads.restype = ctypes.c_int
    lib.fa_oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                  ctypes.c_int, ctypes.c_double, ip, ctypes.c_int]
    lib.fa_oracle_bwd.restype = ctypes.c_int
    lib.fa_oracle_bwd_sample.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                         ctypes.c_int, ctypes.c_double, ip, i64, i64,
                                         i64, lp, i64, lp, dp, dp, dp, ctypes.c_int]
    lib.fa_oracle_bwd_sample.restype = ctypes.c_int
    lib.fa_oracle_decode_paged.argtypes = [dp, dp, dp, ip, ip, dp, dp, i64, i64, i64, i64, i64, i64,
                                           ctypes.c_double, ctypes.c_int]
    lib.fa_oracle_decode_paged.restype = ctypes.c_int
    bp = ctypes.POINTER(ctypes.c_uint8)
    sp = ctypes.POINTER(ctypes.c_int8)
    lib.fa_oracle_fp8_quantize.argtypes = [dp, sp, ctypes.c_int, bp, ip, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.fa_oracle_fp8_quantize.restype = ctypes.c_int
    lib.fa_oracle_fwd_fp8.argtypes = [bp, ip, i64, bp, ip, i64, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_double, ip, ctypes.c_int]
    lib.fa_oracle_fwd_fp8.restype = ctypes.c_int
    lib.fa_oracle_fp8_rotate.argtypes = [dp, sp, ctypes.POINTER(ctypes.c_float), i64, i64]
    lib.fa_oracle_fp8_rotate.restype = ctypes.c_int
    return lib


def _library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            compile_library()
        _lib = load(LIBRARY)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _limits(kv_limit, B: int, N: int):
    if kv_limit is None:
        return None, None
    lim = np.ascontiguousarray(kv_limit, dtype=np.int32)
    if lim.shape != (B, N):
        raise ValueError(f"kv_limit must have shape {(B, N)}, got {lim.shape}")
    return lim, _ptr(lim, ctypes.c_int32)


def attention(q, k, v, causal: bool = False, scale: Optional[float] = None,
              kv_limit=None, nthreads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Every row of attention for q, k, v of shape (B, H, N, d).

    Returns (o, lse): o float64 (B, H, N, d), lse float64 (B, H, N), natural log.
    scale defaults to 1/sqrt(d).
    """
    lib = lib or _library()
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (B, H, N, d) shape")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lim, lim_p = _limits(kv_limit, B, N)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), np.float64)
    rc = lib.fa_oracle_fwd(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                           _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                           B, H, N, d, int(bool(causal)), float(scale), lim_p, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd failed ({rc})")
    return o, lse


def attention_rows(q, k, v, row_ids, causal: bool = False, scale: Optional[float] = None,
                   kv_limit=None, nthreads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected rows only.  row_ids are flat indices (b * H + h) * N + i.

    Returns (o, lse) of shapes (len(row_ids), d) and (len(row_ids),).
    """
    lib = lib or _library()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    lim, lim_p = _limits(kv_limit, B, N)
    o = np.empty((ids.size, d), np.float64)
    lse = np.empty((ids.size,), np.float64)
    rc = lib.fa_oracle_rows(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                            _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                            B, H, N, d, int(bool(causal)), float(scale), lim_p,
                            ids.size, _ptr(ids, ctypes.c_int64), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_rows failed ({rc})")
    return o, lse


def max_threads() -> int:
    return int(_library().fa_oracle_max_threads())


def attention_bwd(q, k, v, dout, causal: bool = False, scale: Optional[float] = None,
                  kv_limit=None, nthreads: int = 0, lib=None, o=None):
    """Gradients of sum(dout * O) with respect to q, k, v, all of shape (B, H, N, d).

    With o (B, H, N, d) given, the row term D_i is <dout_i, o_i> from that
    output instead of the exact one.  Returns (dq, dk, dv) as float64 arrays of
    the same shape.
    """
    lib = lib or _library()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if q.ndim != 4 or any(a.shape != q.shape for a in (k, v, dout)):
        raise ValueError("q, k, v, dout must share one (B, H, N, d) shape")
    o_p = None
    if o is not None:
        o = _f64(o)
        if o.shape != q.shape:
            raise ValueError("o must have the shape of q")
        o_p = _ptr(o, ctypes.c_double)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lim, lim_p = _limits(kv_limit, B, N)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    rc = lib.fa_oracle_bwd(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                           _ptr(dout, ctypes.c_double), o_p, _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                           _ptr(dv, ctypes.c_double), B, H, N, d, int(bool(causal)), float(scale), lim_p,
                           int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd failed ({rc})")
    return dq, dk, dv


def attention_bwd_sample(q, k, v, dout, b: int, h: int, q_rows, k_rows, causal: bool = False,
                         scale: Optional[float] = None, kv_limit=None, nthreads: int = 0, lib=None,
                         o_head=None):
    """Sampled gradients of one head (b, h): dq at query rows q_rows, dk and dv at key rows k_rows.

    Rows are indices within the head.  With o_head (N, d) given, D_i is
    <dout_i, o_head_i>.  Returns (dq, dk, dv) of shapes (len(q_rows), d),
    (len(k_rows), d), (len(k_rows), d).
    """
    lib = lib or _library()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    o_p = None
    if o_head is not None:
        o_head = _f64(o_head)
        if o_head.shape != (N, d):
            raise ValueError("o_head must have shape (N, d)")
        o_p = _ptr(o_head, ctypes.c_double)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lim, lim_p = _limits(kv_limit, B, N)
    qr = np.ascontiguousarray(q_rows, dtype=np.int64)
    kr = np.ascontiguousarray(k_rows, dtype=np.int64)
    dq = np.empty((qr.size, d), np.float64)
    dk = np.empty((kr.size, d), np.float64)
    dv = np.empty((kr.size, d), np.float64)
    rc = lib.fa_oracle_bwd_sample(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                                  _ptr(dout, ctypes.c_double), o_p, B, H, N, d, int(bool(causal)), float(scale),
                                  lim_p,
                                  int(b), int(h), qr.size, _ptr(qr, ctypes.c_int64), kr.size,
                                  _ptr(kr, ctypes.c_int64), _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                                  _ptr(dv, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd_sample failed ({rc})")
    return dq, dk, dv


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: Optional[float] = None,
                 nthreads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention over a paged cache.

    q (B, H, d); k_cache, v_cache (num_pages, H, page_size, d); block_table
    (B, max_pages) int32; seq_lens (B,) int32.  Returns (o, lse): o float64
    (B, H, d), lse float64 (B, H), natural log.  scale defaults to 1/sqrt(d).
    """
    lib = lib or _library()
    q, k_cache, v_cache = _f64(q), _f64(k_cache), _f64(v_cache)
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be (B, H, d) and the caches (num_pages, H, page_size, d)")
    B, H, d = q.shape
    num_pages, Hc, page_size, dc = k_cache.shape
    if (Hc, dc) != (H, d):
        raise ValueError("cache heads and head dim must match q")
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if bt.ndim != 2 or bt.shape[0] != B or lens.shape != (B,):
        raise ValueError("block_table must be (B, max_pages) and seq_lens (B,)")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, d), np.float64)
    lse = np.empty((B, H), np.float64)
    rc = lib.fa_oracle_decode_paged(_ptr(q, ctypes.c_double), _ptr(k_cache, ctypes.c_double),
                                    _ptr(v_cache, ctypes.c_double), _ptr(bt, ctypes.c_int32),
                                    _ptr(lens, ctypes.c_int32), _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                                    B, H, d, page_size, bt.shape[1], num_pages, float(scale), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_decode_paged failed ({rc})")
    return o, lse


def fp8_quantize(x, signs=None, tile_rows: int = 64, nthreads: int = 0, lib=None):
    """E4M3 codes of x (B, H, N, d) with one power-of-two scale per tile of rows.

    With signs (length d, entries +-1) each row is first rotated by the
    unnormalised Hadamard transform of (signs * row); without, rows are encoded
    as they are.  Returns (codes uint8 (B, H, N, d), exps int32 (B, H, ceil(N / tile_rows))).
    """
    lib = lib or _library()
    x = _f64(x)
    B, H, N, d = x.shape
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.int8)
    if sg is not None and sg.shape != (d,):
        raise ValueError("signs must have length d")
    codes = np.empty((B, H, N, d), np.uint8)
    exps = np.empty((B, H, -(-N // tile_rows)), np.int32)
    rc = lib.fa_oracle_fp8_quantize(_ptr(x, ctypes.c_double), None if sg is None else _ptr(sg, ctypes.c_int8),
                                    int(sg is not None), _ptr(codes, ctypes.c_uint8), _ptr(exps, ctypes.c_int32),
                                    B, H, N, d, int(tile_rows), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fp8_quantize failed ({rc})")
    return codes, exps


def attention_fp8(qc, qe, q_tile: int, kc, ke, k_tile: int, v, causal: bool = False, scale: Optional[float] = None,
                  rotated: bool = True, kv_limit=None, nthreads: int = 0, lib=None):
    """Attention on E4M3-coded q and k (codes and per-tile exponents from fp8_quantize) and v.

    rotated: the codes are of Hadamard-rotated rows, so scores are divided by d.
    Returns (o, lse) as fp64 arrays, like attention().
    """
    lib = lib or _library()
    qc = np.ascontiguousarray(qc, dtype=np.uint8)
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    qe = np.ascontiguousarray(qe, dtype=np.int32)
    ke = np.ascontiguousarray(ke, dtype=np.int32)
    v = _f64(v)
    B, H, N, d = qc.shape
    if kc.shape != qc.shape or v.shape != qc.shape:
        raise ValueError("q, k, v must share one (B, H, N, d) shape")
    if qe.shape != (B, H, -(-N // q_tile)) or ke.shape != (B, H, -(-N // k_tile)):
        raise ValueError("exponent arrays do not match the tiles")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lim, lim_p = _limits(kv_limit, B, N)
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    rc = lib.fa_oracle_fwd_fp8(_ptr(qc, ctypes.c_uint8), _ptr(qe, ctypes.c_int32), int(q_tile),
                               _ptr(kc, ctypes.c_uint8), _ptr(ke, ctypes.c_int32), int(k_tile),
                               _ptr(v, ctypes.c_double), _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                               B, H, N, d, int(bool(causal)), float(scale), float(d if rotated else 1), lim_p,
                               int(nthreads))
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd_fp8 failed ({rc})")
    return o, lse


def e4m3_values() -> np.ndarray:
    """fp64 value of every E4M3 code 0..255 (NaN for the two NaN codes), from the format definition."""
    out = np.empty(256)
    for code in range(256):
        s, E, m = code >> 7, (code >> 3) & 15, code & 7
        if (code & 0x7F) == 0x7F:
            out[code] = np.nan
            continue
        v = m * 2.0 ** -9 if E == 0 else (1 + m / 8) * 2.0 ** (E - 7)
        out[code] = -v if s else v
    return out


def fp8_rotate(x, signs, lib=None) -> np.ndarray:
    """The rotation alone: float32 H (signs * row) for every row of x (..., d)."""
    lib = lib or _library()
    x = _f64(x)
    d = x.shape[-1]
    sg = np.ascontiguousarray(signs, dtype=np.int8)
    y = np.empty(x.shape, np.float32)
    rc = lib.fa_oracle_fp8_rotate(_ptr(x, ctypes.c_double), _ptr(sg, ctypes.c_int8), _ptr(y, ctypes.c_float),
                                  x.size // d, d)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fp8_rotate failed ({rc})")
    return y
