"""The correlated-selection workload against the pages' figure.

"3090x3で 314 万コンテキスト", section 5: selections at consecutive steps
overlap by 60-85%, 0.72 on average with the previous step. The committed
AR(1) correlation (tests/golden/correlated_overlap.txt, written by
correlated_overlap.py from the oracle's selections over all 4096 queries of
the 60,000-token-history prefill chunk) must reproduce that average on a
sample of 256 consecutive queries, and the generator must give neighbouring
indexer queries the stated correlation with unit variance.
"""
import os

import numpy as np

import qsa_inputs as qi
from tests.golden import correlated_overlap as co


def _golden():
    vals = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "correlated_overlap.txt")):
        if not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_recorded_overlap_is_the_pages_figure():
    g = _golden()
    assert abs(g["mean_overlap_previous"] - 0.72) <= 0.01
    assert 0.55 <= g["min_overlap_previous"] and g["max_overlap_previous"] <= 0.90


def test_overlap_on_a_sample_of_queries():
    g = _golden()
    pooled, q = co.workload(g["rho"], 256)
    mean = co.overlaps(pooled, q)[0]
    assert abs(mean - 0.72) <= 0.03, mean


def test_ar1_generator_statistics():
    x = qi.bf16_bits_to_f32(qi.ar1_normal_bf16(9, 3, 4000, 128, 0.94859)).astype(np.float64)
    assert abs(x.std() - 1.0) < 0.02
    c = np.mean(np.sum(x[1:] * x[:-1], axis=1) / 128)
    assert abs(c - 0.94859) < 0.01
    x0 = qi.bf16_bits_to_f32(qi.ar1_normal_bf16(9, 3, 4000, 128, 0.0)).astype(np.float64)
    assert abs(np.mean(np.sum(x0[1:] * x0[:-1], axis=1) / 128)) < 0.01
