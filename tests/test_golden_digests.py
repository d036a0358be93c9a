"""The stored oracle digests that bench.py checks its outputs against are
current: recomputing them from the oracle on the seeded workloads gives the
committed file (CPU only)."""
import importlib.util
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def test_workload_digests_are_current():
    spec = importlib.util.spec_from_file_location(
        "make_digests", os.path.join(HERE, "golden", "make_digests.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(mod.OUT) as f:
        stored = json.load(f)
    assert mod.compute() == stored
