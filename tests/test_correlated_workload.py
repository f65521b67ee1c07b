"""The correlated-selection workload against the pages' figure.

"125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 5: selections at consecutive steps
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


def _golden_decode():
    vals = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "correlated_overlap_decode.txt")):
        if not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_decode_workload_overlap_is_the_pages_figure():
    """The 1M-token decode workload (262,080 candidate blocks): the recorded
    rho gives the pages' average overlap with the previous step, within the
    stated 60-85% range, and the union of the last four steps covers more."""
    g = _golden_decode()
    assert abs(g["mean_overlap_previous"] - 0.72) <= 0.015
    assert 0.60 <= g["min_overlap_previous"] and g["max_overlap_previous"] <= 0.85
    assert g["mean_overlap_union4"] > g["mean_overlap_previous"]


def test_decode_workload_overlap_on_a_sample():
    """Recomputed with the oracle for 10 consecutive steps of sequence 2."""
    from tests.golden import correlated_overlap_decode as cod
    g = _golden_decode()
    prev, _ = cod.overlaps(cod.selections(cod.pooled_keys(2), cod.queries(2, g["rho"], 10)))
    assert abs(np.mean(prev) - 0.72) <= 0.05, np.mean(prev)
