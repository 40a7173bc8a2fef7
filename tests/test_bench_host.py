"""Host-side logic of bench.py (no GPU): the single-GPU guard, and the rule that a
stored traffic figure is reported only while the kernel sources it was measured
on are unchanged."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("path", sorted(bench.KERNEL_SOURCES))
def test_kernel_sources_exist(path):
    here = os.path.join(ROOT, "flashattention_forward_attn_amd", "csrc")
    for name in bench.KERNEL_SOURCES[path]:
        assert os.path.isfile(os.path.join(here, name)), name
    assert len(bench._kernel_digest(path)) == 64


@pytest.mark.parametrize("path", sorted(bench.KERNEL_SOURCES))
def test_kernel_sources_cover_the_included_headers(path):
    """A recorded traffic figure is voided by any change to the code its kernel is
    built from, so every header the kernel source includes must be hashed with it.
    Exceptions: fa_launch.h declares host launchers only, and fa_sizes.h (reached
    through it) counts only where the kernel uses one of its constants."""
    here = os.path.join(ROOT, "flashattention_forward_attn_amd", "csrc")
    text = lambda name: open(os.path.join(here, name)).read()

    def includes(name, seen):
        for h in re.findall(r'^#include "([^"]+)"', text(name), re.M):
            if h not in seen:
                seen.add(h)
                includes(h, seen)
        return seen

    main = bench.KERNEL_SOURCES[path][0]
    need = includes(main, set()) - {"fa_launch.h", "fa_sizes.h"}
    sizes = re.findall(r"constexpr\s+\w+\s+(k\w+)\s*=", text("fa_sizes.h"))
    assert sizes
    if any(re.search(rf"\b{n}\b", text(main)) for n in sizes):
        need.add("fa_sizes.h")
    assert need <= set(bench.KERNEL_SOURCES[path]), sorted(need - set(bench.KERNEL_SOURCES[path]))


def test_traffic_reported_only_for_current_sources(tmp_path):
    f = tmp_path / "traffic.json"
    good = {"bytes_per_launch": 123, "kernel_source_sha256": bench._kernel_digest("fused")}
    stale = {"bytes_per_launch": 456, "kernel_source_sha256": "0" * 64}
    f.write_text(json.dumps({"fused": {"w_good": good, "w_stale": stale}}))
    assert bench.load_traffic(str(f), "fused", "w_good") == 123
    assert bench.load_traffic(str(f), "fused", "w_stale") is None
    assert bench.load_traffic(str(f), "fused", "w_missing") is None
    assert bench.load_traffic(str(f), "decode", "w_good") is None
    assert bench.load_traffic(str(tmp_path / "absent.json"), "fused", "w_good") is None



def test_unfused_bytes():
    """S (fp32) and P (bf16) written and read once per head: 12 N^2 bytes, plus
    Q, K, V, O (8 N d) and the fp32 LSE, when N is a multiple of 64."""
    from flashattention_forward_attn_amd import inputs
    w = inputs.WORKLOADS["bf16_causal_b2h32n4096d128"]
    heads = w.B * w.H
    assert bench.unfused_bytes(w) == heads * (12 * w.N ** 2 + 8 * w.N * w.d + 4 * w.N)
    odd = inputs.custom("odd", "f32", 1, 1, 100, 64, False)        # rows padded to 128 keys, fp32 P
    assert bench.unfused_bytes(odd) == 100 * 128 * 16 + 4 * 100 * 64 * 4 + 100 * 4
