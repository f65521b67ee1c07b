"""Pins of the oracle's FP8 (OCP E4M3) functions, against what the format's
definition and arithmetic fix rather than against the oracle's own formulas:

* code values the specification states (largest finite 448 = S.1111.110,
  smallest normal 2^-6 = S.0001.000, largest subnormal 0.875 * 2^-6 =
  S.0000.111, smallest subnormal 2^-9 = S.0000.001, one = S.0111.000, NaN =
  S.1111.111, no infinities), and the ordering of the finite codes;
* rounding checked against a brute-force nearest search over all 254 finite
  values (ties to the even code), including every midpoint;
* quantization checked by its error bound, by the saturation of each
  group's largest magnitude to 448, and on all-zero groups;
* FP8 scores checked with one-hot queries (the score is then one
  dequantized value) and against pure-Python loops on a tiny case.
"""
import numpy as np
import pytest

from oracle import qsa_oracle as orc


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    v = orc.e4m3_to_f64(c)
    keep = np.isfinite(v)
    return c[keep], v[keep]


def test_e4m3_values_stated_by_the_format():
    v = orc.e4m3_to_f64(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0x00, 0x80, 0xFE, 0x88], dtype=np.uint8))
    assert v[0] == 448.0
    assert v[1] == 2.0 ** -6
    assert v[2] == 0.875 * 2.0 ** -6
    assert v[3] == 2.0 ** -9
    assert v[4] == 1.0
    assert v[5] == 0.0 and not np.signbit(v[5])
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -448.0
    assert v[8] == -(2.0 ** -6)
    assert np.all(np.isnan(orc.e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))))
    c, vals = _finite_codes()
    assert c.size == 254 and np.all(np.isfinite(vals))  # no infinities, two NaNs


def test_e4m3_positive_codes_increase():
    v = orc.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    neg = orc.e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -v)


def _brute_nearest(x):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code;
    beyond the largest value, the largest (saturation)."""
    c, v = _finite_codes()
    pos = c < 0x80
    cp, vp = c[pos], v[pos]
    out = []
    for xi in np.atleast_1d(x):
        a = min(abs(xi), 448.0)
        d = np.abs(vp - a)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:
            best = best[(cp[best] & 1) == 0]
        code = int(cp[best[0]])
        if np.signbit(xi):
            code |= 0x80
        out.append(code)
    return np.array(out, dtype=np.uint8)


def test_e4m3_rounding_matches_brute_force():
    _, v = _finite_codes()
    vp = np.sort(np.unique(v[v >= 0]))
    mids = (vp[:-1] + vp[1:]) / 2
    rng = np.random.default_rng(17)
    xs = np.concatenate([
        vp, -vp, mids, -mids, mids * (1 + 1e-12), mids * (1 - 1e-12),
        rng.normal(0, 30, 4000), rng.uniform(-2 ** -5, 2 ** -5, 2000),
        [448.0, 449.0, 463.999, 464.0, 470.0, 1e6, -1e30, 2.0 ** -10, -(2.0 ** -11)],
    ])
    assert np.array_equal(orc.f64_to_e4m3(xs), _brute_nearest(xs))


def test_e4m3_ties_go_to_the_even_code():
    _, v = _finite_codes()
    vp = np.sort(np.unique(v[v >= 0]))
    mids = (vp[:-1] + vp[1:]) / 2
    codes = orc.f64_to_e4m3(mids)
    assert np.all((codes & 1) == 0)


def test_quantize_error_bound_and_saturation():
    rng = np.random.default_rng(5)
    x = orc.bf16_to_f64(orc.f64_to_bf16(rng.normal(0, 1, (300, 128)) * rng.uniform(0.01, 100, (300, 1))))
    codes, scales = orc.quantize_e4m3(x, 128)
    assert scales.dtype == np.float32 and scales.shape == (300, 1)
    deq = orc.dequantize_e4m3(codes, scales, 128)
    s = scales.astype(np.float64)
    # normal range: 4 significant bits, so at most half a step of 2^-3 relative;
    # the subnormal range: half of the 2^-9 step, times the scale; plus the
    # rounding of the fp32 quotient
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - x) <= bound)
    # every group's largest magnitude lands on +-448
    j = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(300), j]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.all(np.abs(orc.e4m3_to_f64(codes)) <= 448.0)


def test_quantize_groups_are_independent():
    rng = np.random.default_rng(6)
    x = orc.bf16_to_f64(orc.f64_to_bf16(rng.normal(0, 1, (7, 512))))
    codes, scales = orc.quantize_e4m3(x, 128)
    for g in range(4):
        c1, s1 = orc.quantize_e4m3(x[:, 128 * g:128 * (g + 1)], 128)
        assert np.array_equal(codes[:, 128 * g:128 * (g + 1)], c1)
        assert np.array_equal(scales[:, g:g + 1], s1)


def test_quantize_zero_group():
    codes, scales = orc.quantize_e4m3(np.zeros((2, 128)), 128)
    assert not np.any(codes) and not np.any(scales)
    assert not np.any(orc.dequantize_e4m3(codes, scales, 128))


def test_fp8_scores_one_hot_and_brute_force():
    rng = np.random.default_rng(7)
    keys = orc.f64_to_bf16(rng.normal(0, 1, (40, 128)))
    codes, scales = orc.fp8_keys(keys)
    assert codes.shape == (40, 128) and scales.shape == (40,)
    deq = orc.dequantize_e4m3(codes, scales[:, None], 128)
    for d in (0, 77, 127):
        q = np.zeros(128, dtype=np.uint16)
        q[d] = 0x3F80  # bf16 1.0
        assert np.array_equal(orc.index_scores_fp8(q, codes, scales, 40), deq[:, d])
    q = orc.f64_to_bf16(rng.normal(0, 1, 128))
    qv = orc.bf16_to_f64(q)
    s = orc.index_scores_fp8(q, codes, scales, 33)
    assert s.shape == (33,)
    for b in range(33):
        tot = 0.0
        for d in range(128):
            tot += float(qv[d]) * float(orc.e4m3_to_f64(codes[b, d])) * float(scales[b])
        assert abs(tot - s[b]) <= 1e-12 * max(1.0, abs(tot))


def test_fp8_relu_scores_brute_force():
    rng = np.random.default_rng(8)
    keys = orc.f64_to_bf16(rng.normal(0, 1, (20, 64)))
    codes, scales = orc.fp8_keys(keys)
    q = orc.f64_to_bf16(rng.normal(0, 1, (4, 64)))
    w = rng.uniform(-1, 1, 4).astype(np.float32)
    s = orc.index_scores_relu_fp8(q, w, codes, scales, 20)
    qv = orc.bf16_to_f64(q)
    for t in range(20):
        tot = 0.0
        for h in range(4):
            dot = sum(float(qv[h, d]) * float(orc.e4m3_to_f64(codes[t, d])) * float(scales[t]) for d in range(64))
            tot += float(w[h]) * max(0.0, dot)
        assert abs(tot - s[t]) <= 1e-12 * max(1.0, abs(tot))


def test_fp8_latent_row_layout_and_bytes():
    rng = np.random.default_rng(9)
    lat = orc.f64_to_bf16(rng.normal(0, 1, (6, 576)))
    codes, scales, rope = orc.fp8_latent(lat)
    assert codes.shape == (6, 512) and scales.shape == (6, 4) and rope.shape == (6, 64)
    # 512 one-byte codes + 4 fp32 scales + 64 bf16 rotary values = 656 bytes
    assert codes[0].nbytes + scales[0].nbytes + rope[0].nbytes == 656
    vals = orc.fp8_latent_values(codes, scales, rope)
    assert np.array_equal(vals[:, 512:], orc.bf16_to_f64(lat[:, 512:]))
    x = orc.bf16_to_f64(lat[:, :512])
    assert np.all(np.abs(vals[:, :512] - x) <= np.abs(x) * 2.0 ** -4 + np.repeat(scales, 128, 1) * 2.0 ** -10)


def test_attend_values_equals_attend_on_bf16_rows():
    rng = np.random.default_rng(10)
    q = orc.f64_to_bf16(rng.normal(0, 1, (16, 256)))
    k = orc.f64_to_bf16(rng.normal(0, 1, (30, 2, 256)))
    v = orc.f64_to_bf16(rng.normal(0, 1, (30, 2, 256)))
    toks = np.array([0, 3, 4, 9, 29])
    o1, l1 = orc.attend(q, k, v, toks, 1 / 16)
    o2, l2 = orc.attend_values(q, orc.bf16_to_f64(k), orc.bf16_to_f64(v), toks, 1 / 16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("bad", [np.inf, np.nan])
def test_e4m3_rounding_rejects_non_finite(bad):
    with pytest.raises(ValueError):
        orc.f64_to_e4m3(np.array([1.0, bad]))


@pytest.mark.parametrize("amax,s", [(448.0, 1.0), (7.0, 1.0 / 64), (3584.0, 8.0)])
def test_quantize_scale_is_amax_over_448(amax, s):
    """Groups whose largest magnitude is 448 * 2^k have the exact scale 2^k,
    so their codes are the plain nearest-even rounding of x / 2^k."""
    rng = np.random.default_rng(11)
    x = orc.bf16_to_f64(orc.f64_to_bf16(rng.uniform(-amax, amax, 128)))
    x[5] = -amax
    codes, scales = orc.quantize_e4m3(x[None, :], 128)
    assert scales[0, 0] == np.float32(s)
    assert np.array_equal(codes[0], _brute_nearest(x / s))
