"""The stored fixture tests/golden/tiny_cached_attention.json still matches the oracle.

The fixture was written by tests/golden/make_golden.py from the oracle alone; a change in the
oracle's arithmetic shows up here first and must name the passage of the pages that
justifies it.
"""

import json
import os

import numpy as np

import oracle

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_cached_attention.json")


def test_fixture_reproduces():
    with open(PATH) as f:
        data = json.load(f)
    assert len(data["cases"]) >= 2
    for case in data["cases"]:
        T = case["T"]
        res = oracle.attend_cached(np.array(case["q"], dtype=np.uint16), np.array(case["k"], dtype=np.uint16),
                                   np.array(case["v"], dtype=np.uint16), np.array(case["bits"]),
                                   np.array(case["mode"]), np.arange(T), case["window"])
        assert res["codes"].tolist() == case["codes"]
        assert res["scale"].view(np.uint32).tolist() == case["scale_f32_bits"]
        assert res["zero"].view(np.uint32).tolist() == case["zero_f32_bits"]
        expect = np.array([[[float.fromhex(x) for x in row] for row in head] for head in case["out_f64_hex"]])
        np.testing.assert_array_equal(res["out"], expect)
