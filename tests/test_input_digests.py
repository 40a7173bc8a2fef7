"""The seeded input generators reproduce the arrays recorded in
tests/golden/input_digests.json (SHA-256 of dtype, shape and bytes), written by
tests/golden/make_input_digests.py.  A deliberate change to a generator rewrites
that file with the script; an accidental one fails here."""
import importlib.util
import json
import os

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
spec = importlib.util.spec_from_file_location("make_input_digests", os.path.join(HERE, "make_input_digests.py"))
mk = importlib.util.module_from_spec(spec)
spec.loader.exec_module(mk)

with open(os.path.join(HERE, "input_digests.json")) as f:
    STORED = json.load(f)


@pytest.mark.parametrize("name", sorted(STORED["workloads"]))
def test_workload_digests(name):
    assert mk.workload_arrays(name) == STORED["workloads"][name]


@pytest.mark.parametrize("name", sorted(STORED["decode"]))
def test_decode_digests(name):
    assert mk.decode_arrays(name) == STORED["decode"][name]


def test_other_digests():
    assert mk.other_arrays() == STORED["other"]


def test_every_generator_is_recorded():
    from flashattention_forward_attn_amd import inputs
    assert set(STORED["workloads"]) == set(inputs.WORKLOADS)
    assert set(STORED["decode"]) == set(inputs.DECODE_WORKLOADS)
