"""CPU checks that the committed measurement evidence matches the code: every benchmark
workload has a rocprofv3 counter summary under profiles/ and an HBM-traffic entry, both taken
from the kernel sources as they are now (bench.py reports the traffic only in that case)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

bench = pytest.importorskip("bench")
profile_counters = pytest.importorskip("profile_counters")


@pytest.mark.parametrize("workload", sorted(bench.WORKLOADS))
def test_workload_profiles_are_current(workload):
    assert workload in profile_counters.KERNEL
    sha = bench.kernel_source_hash(bench.sources_for(workload))
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.txt")
    assert os.path.exists(path), path
    m = re.search(r"kernel source sha1 \(bench.py's kernel_source_hash for this workload\) = ([0-9a-f]{40})",
                  open(path, encoding="utf-8").read())
    assert m and m.group(1) == sha, (workload, "counter summary taken from other kernel sources")
    assert bench.read_traffic(workload) is not None, (workload, "no HBM traffic entry for the current sources")


def test_default_benchmark_trace_is_current():
    path = os.path.join(ROOT, "profiles", f"{bench.DEFAULT}_bench.txt")
    m = re.search(r"kernel source sha1 \(bench.py's kernel_source_hash for this workload\) = ([0-9a-f]{40})",
                  open(path, encoding="utf-8").read())
    assert m and m.group(1) == bench.kernel_source_hash(bench.sources_for(bench.DEFAULT))
