"""Write tests/golden/input_digests.json: SHA-256 of every array the seeded input
generators produce (flashattention_forward_attn_amd.inputs), so that a change to
a generator -- which would silently change every workload -- fails a test.

Run from the repository root:  python tests/golden/make_input_digests.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from flashattention_forward_attn_amd import inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json")


def digest(a) -> str:
    a = np.ascontiguousarray(a)
    h = hashlib.sha256()
    h.update(f"{a.dtype.str}{a.shape}".encode())
    h.update(a.tobytes())
    return h.hexdigest()


def workload_arrays(name):
    w = inputs.WORKLOADS[name]
    x = inputs.generate(w)
    out = {}
    for n in ("q", "k", "v"):
        bits = getattr(x, n + "_bits")
        out[n] = digest(bits if bits is not None else getattr(x, n))
    if x.kv_limit is not None:
        out["kv_limit"] = digest(x.kv_limit)
    if w.dtype == "bf16":
        out["dout"] = digest(inputs.grad_output(w).dout_bits)
    return out


def decode_arrays(name):
    x = inputs.generate_decode(inputs.DECODE_WORKLOADS[name])
    return {n: digest(getattr(x, n)) for n in ("q_bits", "k_bits", "v_bits", "block_table", "seq_lens")}


def other_arrays():
    out = {"fp8_signs_d128": digest(inputs.fp8_signs(128)), "fp8_signs_d64": digest(inputs.fp8_signs(64))}
    for i, a in enumerate(inputs.outlier_qkv(1, 2, 64, 128)):
        out[f"outlier_qkv_{'qkv'[i]}"] = digest(a)
    x = inputs.generate_large()
    for n in ("q_bits", "k_bits", "v_bits", "dout_bits"):
        out["large_" + n] = digest(getattr(x, n))
    xd = inputs.generate_large_decode()
    for n in ("q_bits", "pages", "k_bits", "v_bits", "block_table", "seq_lens"):
        out["large_decode_" + n] = digest(getattr(xd, n))
    return out


def all_digests():
    d = {"workloads": {n: workload_arrays(n) for n in inputs.WORKLOADS},
         "decode": {n: decode_arrays(n) for n in inputs.DECODE_WORKLOADS},
         "other": other_arrays()}
    return d


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(all_digests(), f, indent=1, sort_keys=True)
    print("wrote", OUT)
