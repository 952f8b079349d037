"""Pins for the oracle's fp16 conversion and q8_1 quantization (CPU only).

q8_1 (MMQ page, introduction and "dp4a path Q4_K" section): 32 int8 codes per block with an fp16
scale d and an fp16 sum term s = d * sum(q).  Closed-form blocks live in
tests/golden/q8_1_closed_forms.txt, each worked out by hand.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# fp16 <-> fp32: special cases that reduce to a library routine (numpy's IEEE binary16 casts).
# ---------------------------------------------------------------------------------------------
def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(b) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_float_to_half_matches_numpy_rne():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),     # fp16 subnormal range
        (rng.standard_normal(20000) * 3e4).astype(np.float32),      # near overflow
        (rng.standard_normal(5000) * 1e-8).astype(np.float32),      # underflow to zero
        # exact ties between adjacent fp16 values, in the normal and subnormal ranges
        ((np.arange(1, 2000, dtype=np.float32) + 0.5) * np.float32(2.0 ** -24)),
        ((np.arange(1024, 2048, dtype=np.float32) + 0.5) * np.float32(2.0 ** -10)),
        np.array([65504.0, 65519.996, 65520.0, 65536.0, 1e10, -65520.0, 6.1035156e-05,
                  6.0975552e-05, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 0.0, -0.0,
                  np.inf, -np.inf], dtype=np.float32),
    ])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(v) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


# ---------------------------------------------------------------------------------------------
# q8_1 closed forms
# ---------------------------------------------------------------------------------------------
def _load_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "q8_1_closed_forms.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            val = val.split()
            if key == "case":
                cur = {"name": val[0]}
                cases.append(cur)
            elif key in ("x", "q"):
                arr = np.zeros(32, dtype=np.float64)
                arr[: len(val)] = [float(v) for v in val]
                cur[key] = arr
            else:
                cur[key] = int(val[0], 16)
    return cases


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_q8_1_closed_forms(case):
    x = case["x"].astype(np.float32)[None, :]
    y = oracle.quantize_q8_1(x)[0]
    assert y.shape == (36,)
    d_bits = int(y[0]) | (int(y[1]) << 8)
    s_bits = int(y[2]) | (int(y[3]) << 8)
    q = y[4:36].view(np.int8).astype(np.int64)
    assert np.array_equal(q, case["q"].astype(np.int64)), (q, case["q"])
    assert d_bits == case["d_bits"], hex(d_bits)
    assert s_bits == case["s_bits"], hex(s_bits)


def test_q8_1_block_independence_and_sign_symmetry():
    """Blocks are quantized independently; negating the input negates codes and s, keeps d."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    y = oracle.quantize_q8_1(x)
    y_neg = oracle.quantize_q8_1(-x)
    for r in range(3):
        for b in range(8):
            one = oracle.quantize_q8_1(x[r:r + 1, 32 * b:32 * b + 32])[0]
            assert np.array_equal(one, y[r, 36 * b:36 * b + 36])
            blk, nblk = y[r, 36 * b:36 * b + 36], y_neg[r, 36 * b:36 * b + 36]
            assert np.array_equal(blk[0:2], nblk[0:2])
            assert np.array_equal(blk[4:].view(np.int8), -nblk[4:].view(np.int8))
            s = blk[2:4].copy().view(np.float16)[0]
            ns = nblk[2:4].copy().view(np.float16)[0]
            assert s == -ns


def test_q8_1_properties_random():
    """Properties that hold for every block: |q| <= 127, the largest magnitude maps to +-127, each
    code is within 1/2 (+ fp32 slack) of x/d, and s agrees with d*sum(q) to fp16 precision."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 1024)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    y = oracle.quantize_q8_1(x).reshape(64, 32, 36)
    xb = x.reshape(64, 32, 32).astype(np.float64)
    q = y[:, :, 4:].copy().view(np.int8).astype(np.float64)
    d = y[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    s = y[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    assert np.abs(q).max() <= 127
    amax = np.abs(xb).max(axis=2)
    arg = np.abs(xb).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(q, arg[..., None], 2)[..., 0]) == 127)
    d32 = amax / 127.0
    assert np.all(np.abs(xb / d32[..., None] - q) <= 0.5 + 1e-5)
    assert np.allclose(d, d32, rtol=2 ** -11, atol=0)
    assert np.allclose(s, d32 * q.sum(axis=2), rtol=2 ** -11, atol=2 ** -24)
