"""Pins for the oracle's fp16-activation mode (GP100 MMVQ page, "How" step 1: a power-of-two
prescale per 32 activations with max|y| < 2^15, fp16 values, exact block sums; the accuracy
paragraph under its results table: about 1e-3 relative RMS error against fp64, ten times below
the q8_1 path).  Each pin checks the oracle against something it does not compute itself: numpy's
float16 rounding, a log2-based exponent, math.fsum, exact integer products, scale invariance and
the pages' error figures."""
import math

import numpy as np
import pytest

import oracle
from blockpack import random_q4_K_row, random_q5_K_row, random_q6_K_row, random_q8_0_row, random_q4_0_row

ROWS = {oracle.Q4_K: random_q4_K_row, oracle.Q5_K: random_q5_K_row, oracle.Q6_K: random_q6_K_row,
        oracle.Q8_0: random_q8_0_row, oracle.Q4_0: random_q4_0_row}


def _weights(qtype, rows, k, seed):
    rng = np.random.default_rng(seed)
    return np.concatenate([np.frombuffer(ROWS[qtype](rng, k)[0], np.uint8) for _ in range(rows)])


def _wide_x(n, k, seed):
    """Blocks spanning many binades, zeros, an all-zero block, fp32 extremes."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, k)) * 2.0 ** rng.integers(-40, 40, (n, k // 32)).repeat(32, axis=1)
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = np.float32(1e-45)                # fp32 subnormals
    x[0, 64] = np.float32(3.0e38)                  # near fp32 max: e < 0
    x[0, 96:128] = 2.0 ** 14                       # amax exactly 2^14 -> e = 0
    x[0, 128:160] = -(2.0 ** 15)                   # amax exactly 2^15 -> e = -1
    return x


def _exponent_ref(xb):
    amax = float(np.abs(xb.astype(np.float64)).max())
    return 0 if amax == 0.0 else 14 - math.floor(math.log2(amax))


def test_encoder_exponent_and_fp16_rounding_against_numpy():
    x = _wide_x(3, 512, 1)
    y, e, s = oracle.f16act_encode(x)
    for c in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            xb = x[c, 32 * b:32 * b + 32]
            assert e[c, b] == _exponent_ref(xb), (c, b)
            ref = np.ldexp(xb.astype(np.float64), int(e[c, b])).astype(np.float16)   # numpy: RNE
            assert np.array_equal(y[c, 32 * b:32 * b + 32], ref.view(np.uint16)), (c, b)
            vals = y[c, 32 * b:32 * b + 32].view(np.float16).astype(np.float64)
            if xb.any():
                assert 2.0 ** 14 <= np.abs(vals).max() <= 2.0 ** 15      # prescale bound (rounding may reach 2^15)
            assert s[c, b] == math.fsum(vals)


def test_encoder_ties_round_to_even():
    # after the prescale (amax 2^14 -> e = 0) the fp16 spacing in [2^10, 2^11) is 1: x.5 ties go to even
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2.0 ** 14
    x[0, 1:5] = [1024.5, 1025.5, 1026.5, -1027.5]
    y, e, _ = oracle.f16act_encode(x)
    assert e[0, 0] == 0
    assert list(y[0, 1:5].view(np.float16).astype(np.float64)) == [1024.0, 1026.0, 1026.0, -1028.0]


@pytest.mark.parametrize("qtype", sorted(ROWS))
def test_product_exact_for_fp16_exact_activations(qtype):
    """Activations that are integers below 2^11 survive the encoder exactly (a power-of-two scale
    keeps their 11 significant bits), so the product is the fp64 W.x rounded once to fp32."""
    rows, k, n = 5, 512, 3
    w = _weights(qtype, rows, k, 10 + qtype)
    rng = np.random.default_rng(20 + qtype)
    x = rng.integers(-2047, 2048, (n, k)).astype(np.float32) * np.float32(2.0 ** -7)
    got = oracle.matmul_f16act(qtype, w, rows, k, x)
    ref = (x.astype(np.float64) @ oracle.dequantize(qtype, w, rows, k).T).astype(np.float32)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("j", [-30, -3, 5, 40])
def test_product_scales_exactly_with_powers_of_two(j):
    qtype, rows, k = oracle.Q4_K, 4, 512
    w = _weights(qtype, rows, k, 31)
    x = np.random.default_rng(32).standard_normal((2, k)).astype(np.float32)
    a = oracle.matmul_f16act(qtype, w, rows, k, x)
    b = oracle.matmul_f16act(qtype, w, rows, k, np.ldexp(x, j).astype(np.float32))
    assert np.array_equal(np.ldexp(a.astype(np.float64), j), b.astype(np.float64))


@pytest.mark.parametrize("qtype", sorted(ROWS))
def test_error_band_against_fp64_and_q8_1(qtype):
    """Relative RMS error against fp64 with unquantized activations: the page quotes 1.1e-3 for
    the fp16 mode and 1.2e-2 for the q8_1 path on a real tensor; random data lands in the same
    places (fp16 keeps 11 bits, q8_1 about 8)."""
    rows, k, n = 64, 2048, 4
    w = _weights(qtype, rows, k, 40 + qtype)
    x = np.random.default_rng(41).standard_normal((n, k)).astype(np.float32)
    exact = x.astype(np.float64) @ oracle.dequantize(qtype, w, rows, k).T
    def rel(y):
        return math.sqrt(((y - exact) ** 2).sum() / (exact ** 2).sum())
    e16 = rel(oracle.matmul_f16act(qtype, w, rows, k, x).astype(np.float64))
    e8 = rel(oracle.matmul_q8_1(qtype, w, rows, k, oracle.quantize_q8_1(x), n).astype(np.float64))
    assert 5e-5 < e16 < 2e-3
    assert e8 > 10 * e16
