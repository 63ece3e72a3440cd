"""The seeded input generator (synth/): every workload's inputs against their
recorded SHA-256 (tests/golden/synth_sha256.json, written by
write_synth_sha256.py beside it), and values independent of the thread count.
The generator holds none of the quantizer's arithmetic; these pins keep the
inputs of every parity test and of the benchmark fixed."""
import hashlib
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "synth_sha256.json")


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_inputs_match_recorded_sha256(name):
    with open(GOLD) as f:
        want = json.load(f)["workloads"][name]
    got = {k: hashlib.sha256(v.tobytes()).hexdigest() for k, v in synth.workload(name).inputs().items()}
    assert got == want


def test_values_do_not_depend_on_the_thread_count():
    """Normal draws, uniform outliers, t3 outliers and uniforms with 1, 3 and
    16 threads (chunk bounds fall at different elements each time)."""
    shape = (1531, 2347)  # 3.6M elements: more than one chunk per thread
    runs = []
    try:
        for n in (1, 3, 16):
            synth.set_threads(n)
            a = synth.normal_bf16(9, synth.T_X, shape, 1.0)
            synth.add_outliers_uniform(a, 9, 0.01, 50.0, 300.0)
            b = synth.normal_bf16(10, synth.T_X, shape, 1.0)
            synth.add_outliers_t3(b, 10, 0.001, 20.0)
            runs.append((a, b, synth.uniform(9, synth.T_ROWS, 1 << 20)))
    finally:
        synth.set_threads(None)
    for other in runs[1:]:
        for x, y in zip(runs[0], other):
            assert np.array_equal(x, y)
