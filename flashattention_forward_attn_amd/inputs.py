"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the HIP path's callers and by the oracle's callers.
It holds random draws, the fp32 -> bf16 round-to-nearest-even conversion and
the workload table, and none of the attention arithmetic.

Tensor layout follows the [b, h, seq, d] shape used for Q, K and V in
"谁偷走了 5090 的算力和显存" (the attention section, eager attention in five
steps): contiguous, row-major, d fastest.

Draw order for every workload: Q, K, V (each a float64 standard normal of
shape (B, H, N, d), cast to float32), then, for the key-padding workload, the
per-batch valid lengths, the batch item that gets a fully masked query block,
and that block's start.  All draws come from ``numpy.random.default_rng(seed)``.

For the backward pass, the upstream gradient dO (same shape as O, standard
normal, float64 cast to float32, then rounded like the other inputs) comes from
its own stream, ``numpy.random.default_rng([seed, 1])``, so the forward inputs
are unchanged by it.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

# Rows of the query block that the key-padding workload masks out entirely.
MASKED_QUERY_BLOCK = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN inputs are not expected (the generators never produce them).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "bf16" or "f32"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    qk_mult: float = 1.0        # Q and K draws are multiplied by this before rounding
    v_dist: str = "normal"      # "normal": N(0,1); "uniform": U(-1, 1)
    key_padding: bool = False   # per-batch valid key length plus one fully masked query block
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def flops(self) -> float:
        """Nominal forward FLOPs: two N x N x d contractions per head, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Nominal backward FLOPs: five N x N x d contractions per head (the
        recomputed scores, dV, dP, dQ and dK), halved when causal."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def describe(self) -> dict:
        return dataclasses.asdict(self)


# The five workloads the method is measured on (fp32 single head; bf16
# non-causal; bf16 causal; bf16 causal long context; bf16 key-padding stress).
WORKLOADS = {
    "f32_b1h1n256d64": Workload("f32_b1h1n256d64", "f32", 1, 1, 256, 64, False),
    "bf16_b4h16n2048d64": Workload("bf16_b4h16n2048d64", "bf16", 4, 16, 2048, 64, False),
    "bf16_causal_b2h32n4096d128": Workload("bf16_causal_b2h32n4096d128", "bf16", 2, 32, 4096, 128, True),
    "bf16_causal_b1h16n16384d128": Workload("bf16_causal_b1h16n16384d128", "bf16", 1, 16, 16384, 128, True),
    "bf16_keypad_b8h32n1024d128": Workload("bf16_keypad_b8h32n1024d128", "bf16", 8, 32, 1024, 128, False,
                                           qk_mult=8.0, v_dist="uniform", key_padding=True),
}


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    q, k, v are fp32 arrays of shape (B, H, N, d).  For bf16 workloads every
    value is exactly representable in bf16 and ``*_bits`` hold the bf16 bit
    patterns the device receives; for fp32 workloads ``*_bits`` are None.
    kv_limit is None or an int32 array of shape (B, N): query row i of batch
    item b may attend to keys j < kv_limit[b, i].
    """
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kv_limit: Optional[np.ndarray]
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    lengths: Optional[np.ndarray] = None
    masked_batch: Optional[int] = None
    masked_q0: Optional[int] = None

    def digests(self) -> dict:
        out = {}
        for name in ("q", "k", "v", "kv_limit"):
            a = getattr(self, name)
            if a is not None:
                out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs (see the module docstring for the draw order)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = (rng.standard_normal(shape).astype(np.float32)) * np.float32(w.qk_mult)
    k = (rng.standard_normal(shape).astype(np.float32)) * np.float32(w.qk_mult)
    if w.v_dist == "normal":
        v = rng.standard_normal(shape).astype(np.float32)
    elif w.v_dist == "uniform":
        v = rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    else:
        raise ValueError(f"unknown v_dist {w.v_dist!r}")

    kv_limit = lengths = masked_batch = masked_q0 = None
    if w.key_padding:
        lengths = rng.integers(1, w.N + 1, size=w.B).astype(np.int32)
        masked_batch = int(rng.integers(0, w.B))
        n_blocks = -(-w.N // MASKED_QUERY_BLOCK)
        masked_q0 = int(rng.integers(0, n_blocks)) * MASKED_QUERY_BLOCK
        kv_limit = np.repeat(lengths[:, None], w.N, axis=1).astype(np.int32)
        kv_limit[masked_batch, masked_q0:masked_q0 + MASKED_QUERY_BLOCK] = 0

    if w.dtype == "bf16":
        qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        return Inputs(w, bf16_to_f32(qb), bf16_to_f32(kb), bf16_to_f32(vb), kv_limit,
                      qb, kb, vb, lengths, masked_batch, masked_q0)
    if w.dtype == "f32":
        return Inputs(w, q, k, v, kv_limit, None, None, None, lengths, masked_batch, masked_q0)
    raise ValueError(f"unknown dtype {w.dtype!r}")


def custom(name: str, dtype: str, B: int, H: int, N: int, d: int, causal: bool, **kw) -> Workload:
    """A workload of any shape, for parity sweeps over odd sizes."""
    return Workload(name, dtype, B, H, N, d, causal, **kw)


def random_kv_limit(B: int, N: int, seed: int, kind: str) -> np.ndarray:
    """Per-row key limits for mask sweeps: 'random' (each row uniform in [0, N]),
    'zeros' (every row fully masked), 'some_zero' (random, with every fifth row 0),
    'out_of_range' (uniform in [-N, 2N], with the int32 extremes every seventh and
    eleventh row: the API clamps negative limits to 0 and limits past N to N)."""
    rng = np.random.default_rng(seed)
    if kind == "zeros":
        return np.zeros((B, N), np.int32)
    if kind == "out_of_range":
        lim = rng.integers(-N, 2 * N + 1, size=(B, N)).astype(np.int32)
        lim[:, ::7] = np.iinfo(np.int32).min
        lim[:, 3::11] = np.iinfo(np.int32).max
        return lim
    lim = rng.integers(0, N + 1, size=(B, N)).astype(np.int32)
    if kind == "some_zero":
        lim[:, ::5] = 0
    elif kind != "random":
        raise ValueError(kind)
    return lim


@dataclasses.dataclass
class GradOutput:
    dout: np.ndarray                       # float32 values (exactly bf16 values for bf16 workloads)
    dout_bits: Optional[np.ndarray] = None  # uint16 bf16 bits (bf16 workloads)

    def digest(self) -> str:
        return hashlib.sha256(np.ascontiguousarray(self.dout).tobytes()).hexdigest()


def grad_output(w: Workload, seed: Optional[int] = None) -> GradOutput:
    """The upstream gradient dO for the backward pass (its own random stream)."""
    rng = np.random.default_rng([w.seed if seed is None else seed, 1])
    g = rng.standard_normal((w.B, w.H, w.N, w.d)).astype(np.float32)
    if w.dtype == "bf16":
        bits = bf16_bits(g)
        return GradOutput(bf16_to_f32(bits), bits)
    if w.dtype == "f32":
        return GradOutput(g, None)
    raise ValueError(f"unknown dtype {w.dtype!r}")


# ---------------------------------------------------------------- paged decode
#
# Decode: one query per sequence over its cached keys, the cache cut into pages
# of 16 tokens reached through a per-sequence block table.  Draw order from
# ``numpy.random.default_rng([seed, 2])``: the sequence lengths (uniform in
# [1, max_len]), the permutation that scatters the needed pages (plus a spare
# tenth) over the pool, q, then k_cache and v_cache (float32 standard normal
# draws over the whole pool, 256 pages per draw, unused slots included), all
# rounded to bf16.
# Block-table entries past a sequence's pages point at page 0.

DECODE_PAGE = 16


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    d: int
    max_len: int        # tokens reserved per sequence (max_pages * 16)
    seed: int = 0

    @property
    def max_pages(self) -> int:
        return -(-self.max_len // DECODE_PAGE)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


@dataclasses.dataclass
class DecodeInputs:
    workload: DecodeWorkload
    q: np.ndarray            # float32 (B, H, d), bf16 values
    k_cache: np.ndarray      # float32 (num_pages, H, 16, d), bf16 values
    v_cache: np.ndarray
    block_table: np.ndarray  # int32 (B, max_pages)
    seq_lens: np.ndarray     # int32 (B,)
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of the cached keys and values the sequences actually use (bf16)."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.workload.H * self.workload.d * 2 * 2

    def flops(self) -> float:
        """Two length x d products per (sequence, head)."""
        return 4.0 * float(self.seq_lens.astype(np.int64).sum()) * self.workload.H * self.workload.d


# Decode workloads: the page's scenario (space reserved for 2048 tokens per
# sequence, each sequence at its own length), and a long-context variant.
DECODE_WORKLOADS = {
    "decode_b64h32d128_len2048": DecodeWorkload("decode_b64h32d128_len2048", 64, 32, 128, 2048),
    "decode_b8h16d64_len16384": DecodeWorkload("decode_b8h16d64_len16384", 8, 16, 64, 16384),
}


def generate_decode(w: DecodeWorkload, seed: Optional[int] = None, lens=None) -> DecodeInputs:
    rng = np.random.default_rng([w.seed if seed is None else seed, 2])
    drawn = rng.integers(1, w.max_len + 1, size=w.B).astype(np.int32)
    seq_lens = drawn if lens is None else np.asarray(lens, np.int32)
    need = [-(-max(int(n), 0) // DECODE_PAGE) for n in seq_lens]
    total = sum(need)
    num_pages = max(1, total + total // 10)
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.zeros((w.B, w.max_pages), np.int32)
    at = 0
    for b, n in enumerate(need):
        block_table[b, :n] = perm[at:at + n]
        at += n
    qb = bf16_bits(rng.standard_normal((w.B, w.H, w.d), dtype=np.float32))
    cache_bits = []
    for _ in range(2):  # k_cache, then v_cache, drawn 256 pages at a time
        bits = np.empty((num_pages, w.H, DECODE_PAGE, w.d), np.uint16)
        for p0 in range(0, num_pages, 256):
            n = min(256, num_pages - p0)
            bits[p0:p0 + n] = bf16_bits(rng.standard_normal((n, w.H, DECODE_PAGE, w.d), dtype=np.float32))
        cache_bits.append(bits)
    kb, vb = cache_bits
    return DecodeInputs(w, bf16_to_f32(qb), bf16_to_f32(kb), bf16_to_f32(vb), block_table, seq_lens, qb, kb, vb)


def fp8_signs(d: int, seed: int = 0) -> np.ndarray:
    """The random +-1 vector of the FP8 path's incoherent processing (one per head
    dimension, shared by Q and K): ``default_rng([seed, 3])``."""
    return np.random.default_rng([seed, 3]).choice(np.array([-1, 1], np.int8), size=d)


def outlier_qkv(B: int, H: int, N: int, d: int, seed: int = 0, n_out: int = 4, mult: float = 20.0):
    """bf16-exact Q, K, V with a few outlier feature columns in Q and K (the FP8
    accuracy workload): normal draws times 0.25, the chosen columns times mult."""
    rng = np.random.default_rng([seed, 4])
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    cols = rng.choice(d, n_out, replace=False)
    q[..., cols] *= mult
    k[..., cols] *= mult
    q *= 0.25
    k *= 0.25
    return tuple(bf16_to_f32(bf16_bits(a)) for a in (q, k, v))


# ---------------------------------------------------------------- tensors beyond 2^31 elements
#
# A [B, H, N, d] shape whose tensors hold more than 2^31 elements, mostly zero:
# only the listed (batch, head) pairs carry data, drawn from
# ``default_rng([seed, 5])`` in the order Q, K, V, dO (float32 standard normal,
# rounded to bf16), each of shape [len(heads), N, d].  Every row sees the first
# `limit` keys (kv_limit = limit for all rows).  The last two listed pairs start
# past element 2^31, so a 32-bit element offset would miss them.

@dataclasses.dataclass(frozen=True)
class LargeCase:
    B: int = 2
    H: int = 8256
    N: int = 1024
    d: int = 128
    limit: int = 64
    heads: tuple = (0, 8000, 16384, 16511)   # flattened b * H + h
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def elements(self) -> int:
        return self.B * self.H * self.N * self.d


@dataclasses.dataclass
class LargeInputs:
    case: LargeCase
    q_bits: np.ndarray     # uint16 [S, N, d] for the listed heads
    k_bits: np.ndarray
    v_bits: np.ndarray
    dout_bits: np.ndarray

    def values(self, name: str) -> np.ndarray:
        """float64 values of one of q, k, v, dout as [1, S, N, d]."""
        return bf16_to_f32(getattr(self, name + "_bits")).astype(np.float64)[None]


def generate_large(case: LargeCase = LargeCase()) -> LargeInputs:
    rng = np.random.default_rng([case.seed, 5])
    shape = (len(case.heads), case.N, case.d)
    bits = [bf16_bits(rng.standard_normal(shape).astype(np.float32)) for _ in range(4)]
    return LargeInputs(case, *bits)


# A paged cache whose pool holds more than 2^31 elements per cache, mostly zero:
# the sequences' pages are the last pages of the pool (past element 2^31), in a
# shuffled order.  Draw order from ``default_rng([seed, 6])``: the order of the
# used pages, q (B, H, d), then the used pages of k and v (float32 standard
# normal, rounded to bf16).  Block-table entries past a sequence's pages are 0.

@dataclasses.dataclass(frozen=True)
class LargeDecodeCase:
    H: int = 32
    d: int = 128
    num_pages: int = 33000
    seq_lens: tuple = (37, 300)
    seed: int = 0

    @property
    def B(self) -> int:
        return len(self.seq_lens)

    @property
    def max_pages(self) -> int:
        return max(-(-n // DECODE_PAGE) for n in self.seq_lens)

    def page_elements(self) -> int:
        return self.H * DECODE_PAGE * self.d


@dataclasses.dataclass
class LargeDecodeInputs:
    case: LargeDecodeCase
    q_bits: np.ndarray        # uint16 (B, H, d)
    pages: np.ndarray         # int32: pool index of each used page, in table order
    k_bits: np.ndarray        # uint16 (len(pages), H, 16, d), the used pages only
    v_bits: np.ndarray
    block_table: np.ndarray   # int32 (B, max_pages), pool indices
    seq_lens: np.ndarray      # int32 (B,)


def generate_large_decode(case: LargeDecodeCase = LargeDecodeCase()) -> LargeDecodeInputs:
    rng = np.random.default_rng([case.seed, 6])
    counts = [-(-n // DECODE_PAGE) for n in case.seq_lens]
    used = sum(counts)
    pages = (case.num_pages - used + rng.permutation(used)).astype(np.int32)
    q = bf16_bits(rng.standard_normal((case.B, case.H, case.d)).astype(np.float32))
    shape = (used, case.H, DECODE_PAGE, case.d)
    k = bf16_bits(rng.standard_normal(shape).astype(np.float32))
    v = bf16_bits(rng.standard_normal(shape).astype(np.float32))
    table = np.zeros((case.B, case.max_pages), np.int32)
    at = 0
    for b, n in enumerate(counts):
        table[b, :n] = pages[at:at + n]
        at += n
    return LargeDecodeInputs(case, q, pages, k, v, table, np.asarray(case.seq_lens, np.int32))
