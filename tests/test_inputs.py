"""Seeded input generator: published SplitMix64 outputs and table properties."""
import numpy as np

import qsa_inputs as qi


def test_splitmix64_reference_outputs():
    # First outputs of SplitMix64 started at state 1234567 (the test vector of
    # the reference C implementation by S. Vigna).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    state = np.uint64(1234567)
    with np.errstate(over="ignore"):
        got = [int(qi.mix64(state + np.uint64(i + 1) * np.uint64(qi.G))) for i in range(5)]
    assert got == want


def test_words_are_index_addressable():
    a = qi.normal_bf16(3, 9, 0, 1000)
    idx = np.array([999, 0, 517, 4, 3, 2, 1], dtype=np.uint64)
    assert np.array_equal(qi.normal_bf16(3, 9, 0, index=idx), a[idx.astype(np.int64)])
    assert np.array_equal(qi.normal_bf16(3, 9, 500, 500), a[500:])


def test_normal_table_is_symmetric_standard_normal():
    t = qi.bf16_bits_to_f32(qi.normal_table()).astype(np.float64)
    assert np.all(np.diff(t) >= 0)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1.0) < 1e-3


def test_streams_differ():
    a = qi.normal_bf16(1, qi.stream_id(0, 0, "k"), 0, 64)
    b = qi.normal_bf16(1, qi.stream_id(0, 0, "v"), 0, 64)
    c = qi.normal_bf16(1, qi.stream_id(1, 0, "k"), 0, 64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
