"""Pins for the oracle's integer sub-block dots and the fp64 scale combine (CPU only).

MMQ page, "dp4a path Q4_K" section: per q8_1 block an integer dot of unsigned nibbles and int8
codes, then d*sum(d8*sc*sumi) - dmin*sum(s8*m).  "Q6_K dot" section: two 16-value sub-blocks per
q8_1 block, each with its own int8 scale, d6*sum d8*(sc0*x + sc1*y).  "write-back" section: the
integer part is exact, the error comes from the float scale arithmetic.
"""
import numpy as np
import pytest

import oracle
import synth
from blockpack import (pack_q4_K, random_q4_0_row, random_q4_K_row, random_q5_K_row, random_q6_K_row, random_q8_0_row,
                       random_q3_K_row, random_iq4_xs_row,
                       weight_codes,
                       q8_1_codes, q8_1_scales)

ROWGEN = {oracle.Q4_K: random_q4_K_row, oracle.Q5_K: random_q5_K_row, oracle.Q6_K: random_q6_K_row,
          oracle.Q8_0: random_q8_0_row, oracle.Q4_0: random_q4_0_row, oracle.Q3_K: random_q3_K_row,
          oracle.IQ4_XS: random_iq4_xs_row}
ALL_TYPES = [oracle.Q4_K, oracle.Q5_K, oracle.Q6_K, oracle.Q8_0, oracle.Q4_0, oracle.Q3_K, oracle.IQ4_XS]


def _rows(qtype, rows, k, rng):
    data, fields = zip(*[ROWGEN[qtype](rng, k) for _ in range(rows)])
    return np.stack(data), list(fields)


@pytest.mark.parametrize("qtype", ALL_TYPES)
def test_subdots_brute_force(qtype):
    """Integer dots from the encoder's own codes and the q8_1 bytes, summed in Python ints."""
    rng = np.random.default_rng(20)
    rows, k, n = 5, 512, 3
    w, fields = _rows(qtype, rows, k, rng)
    x = rng.standard_normal((n, k)).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    D = oracle.subdots(qtype, w, rows, k, xq, n)
    sub = 16 if qtype in (oracle.Q6_K, oracle.Q3_K) else 32
    assert D.shape == (n, rows, k // sub)
    for c in range(n):
        qa = q8_1_codes(xq[c])
        for r in range(rows):
            qw = weight_codes(qtype, fields[r])
            for b in range(k // sub):
                expect = sum(int(qw[i]) * int(qa[i]) for i in range(b * sub, (b + 1) * sub))
                assert D[c, r, b] == expect


def _min_correction(qtype, fields, xq_row):
    """Q4_K / Q5_K: the method uses the stored fp16 s where exact dequantization has d*sum(q); the
    difference per sub-block is dmin*m*(s - d*sum(q)).  Returns sum over sub-blocks."""
    if qtype not in (oracle.Q4_K, oracle.Q5_K):
        return 0.0
    d, s = q8_1_scales(xq_row)
    qa = q8_1_codes(xq_row).reshape(-1, 32)
    corr = 0.0
    for sb, (_, dmin, _, m, _) in enumerate(fields):
        for j in range(8):
            b = 8 * sb + j
            corr += dmin * m[j] * (s[b] - d[b] * qa[b].sum())
    return corr


@pytest.mark.parametrize("qtype", ALL_TYPES)
@pytest.mark.parametrize("shape", [(7, 256, 3), (16, 1024, 5), (3, 512, 17)])
def test_matches_fp64_dequantize_then_multiply(qtype, shape):
    """Y equals the fp64 product of the dequantized weights and dequantized q8_1 activations
    (plus, for Q4_K, the exactly computable stored-s correction), up to the final fp32 rounding."""
    rows, k, n = shape
    rng = np.random.default_rng(21)
    w, fields = _rows(qtype, rows, k, rng)
    x = rng.standard_normal((n, k)).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    y = oracle.matmul_q8_1(qtype, w, rows, k, xq, n).astype(np.float64)
    W = oracle.dequantize(qtype, w, rows, k)
    X, _, _ = oracle.dequantize_q8_1(xq, n, k)
    Y64 = X @ W.T
    for c in range(n):
        for r in range(rows):
            expect = Y64[c, r] - _min_correction(qtype, fields[r], xq[c])
            scale = np.linalg.norm(W[r]) * np.linalg.norm(X[c])
            assert abs(y[c, r] - expect) <= 2.0 ** -23 * abs(expect) + 1e-12 * scale, (c, r)


@pytest.mark.parametrize("j", range(8))
def test_q4_K_per_subblock_identity(j):
    """Only sub-block j carries scale and min: Y equals d*sc*d_a*D - dmin*m*s for that block, which
    is the fp64 dequantized dot over those 32 values minus dmin*m*(s - d_a*sum(q_a))."""
    rng = np.random.default_rng(30 + j)
    sc = np.zeros(8, int); m = np.zeros(8, int)
    sc[j], m[j] = rng.integers(1, 64), rng.integers(1, 64)
    q = rng.integers(0, 16, 256)
    blk = pack_q4_K(0.0137, 0.0071, sc, m, q)
    x = rng.standard_normal((1, 256)).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    y = float(oracle.matmul_q8_1(oracle.Q4_K, blk, 1, 256, xq, 1)[0, 0])
    W = oracle.dequantize(oracle.Q4_K, blk, 1, 256)[0]
    X, d, s = oracle.dequantize_q8_1(xq, 1, 256)
    qa = q8_1_codes(xq[0])[32 * j:32 * j + 32]
    dmin = float(np.float16(0.0071))
    dot = float(np.dot(W[32 * j:32 * j + 32], X[0, 32 * j:32 * j + 32]))
    expect = dot - dmin * m[j] * (s[0, j] - d[0, j] * qa.sum())
    assert abs(y - expect) <= 2.0 ** -23 * abs(expect) + 1e-15


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K, oracle.Q8_0])
def test_quantization_noise_band(qtype):
    """Against UNquantized N(0,1) activations the q8_1 product carries the activation rounding
    noise: relative RMS near (amax/127)/sqrt(12) / rms(x) ~ 7e-3, and below the 1.2e-2 the GP100
    patch page reports for the q8_1 path on a real tensor ("Result" section)."""
    rng = np.random.default_rng(40)
    rows, k, n = 64, 1024, 8
    w = synth.gen_weights(qtype, rows, k, rng)
    x = rng.standard_normal((n, k)).astype(np.float32)
    y = oracle.matmul(qtype, w, rows, k, x).astype(np.float64)
    W = oracle.dequantize(qtype, w, rows, k)
    ref = x.astype(np.float64) @ W.T
    rel = np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert 2e-3 < rel < 1.2e-2, rel


def test_sampled_outputs_equal_full():
    rng = np.random.default_rng(50)
    for qtype in (oracle.Q4_K, oracle.Q6_K, oracle.Q8_0):
        w = synth.gen_weights(qtype, 40, 512, rng)
        xq = oracle.quantize_q8_1(rng.standard_normal((6, 512)).astype(np.float32))
        y = oracle.matmul_q8_1(qtype, w, 40, 512, xq, 6)
        cols = rng.integers(0, 6, 100); rws = rng.integers(0, 40, 100)
        got = oracle.matmul_q8_1_at(qtype, w, 40, 512, xq, 6, cols, rws)
        assert np.array_equal(got, y[cols, rws])


def test_matmul_is_quantize_then_matmul_q8_1():
    rng = np.random.default_rng(51)
    w = synth.gen_weights(oracle.Q4_K, 8, 512, rng)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    assert np.array_equal(oracle.matmul(oracle.Q4_K, w, 8, 512, x),
                          oracle.matmul_q8_1(oracle.Q4_K, w, 8, 512, oracle.quantize_q8_1(x), 3))


@pytest.mark.parametrize("x_per_tok", [1, 3])
def test_matmul_id_is_loop_of_dense(x_per_tok):
    """MoE: each (token, slot) output row is the dense product with its expert's matrix and its
    activation row; an id outside [0, n_exp) is skipped, counted, and its row left untouched."""
    rng = np.random.default_rng(60)
    n_exp, rows, k, n_tok, top_k = 5, 12, 256, 7, 3
    w = synth.gen_weights(oracle.Q6_K, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok * x_per_tok, k)).astype(np.float32)
    ids = rng.integers(0, n_exp, (n_tok, top_k)).astype(np.int32)
    ids[2, 1] = n_exp          # invalid
    ids[4, 0] = -1             # invalid
    y, bad = oracle.matmul_id(oracle.Q6_K, w, n_exp, rows, k, x, x_per_tok, ids)
    assert bad == 2
    rb = oracle.row_bytes(oracle.Q6_K, k)
    wm = w.reshape(n_exp, rows * rb)
    for t in range(n_tok):
        for s in range(top_k):
            e = ids[t, s]
            if not 0 <= e < n_exp:
                assert np.all(np.isnan(y[t, s]))
                continue
            xr = x[t * x_per_tok + (s if x_per_tok > 1 else 0)][None, :]
            ref = oracle.matmul(oracle.Q6_K, wm[e], rows, k, xr)[0]
            assert np.array_equal(y[t, s], ref)


def test_q6_K_folded_subdots_brute_force():
    """sc[2b]*D[2b] + sc[2b+1]*D[2b+1] per q8_1 block, from the encoder's own scales and codes."""
    rng = np.random.default_rng(70)
    rows, k, n = 4, 512, 2
    w, fields = _rows(oracle.Q6_K, rows, k, rng)
    xq = oracle.quantize_q8_1(rng.standard_normal((n, k)).astype(np.float32))
    F = oracle.subdots_q6_K_folded(w, rows, k, xq, n)
    for c in range(n):
        qa = q8_1_codes(xq[c])
        for r in range(rows):
            qw = weight_codes(oracle.Q6_K, fields[r])
            sc = np.concatenate([f[1] for f in fields[r]])
            for b in range(k // 32):
                expect = sum(int(sc[v // 16]) * int(qw[v]) * int(qa[v]) for v in range(32 * b, 32 * b + 32))
                assert F[c, r, b] == expect


def test_q3_K_folded_subdots_brute_force():
    """(sc[2b]-32)*D[2b] + (sc[2b+1]-32)*D[2b+1] per q8_1 block, D over the codes q - 4, from the
    encoder's own scales and codes (GP100 page, "How" step 3: the -4 offset)."""
    rng = np.random.default_rng(71)
    rows, k, n = 4, 512, 2
    w, fields = _rows(oracle.Q3_K, rows, k, rng)
    xq = oracle.quantize_q8_1(rng.standard_normal((n, k)).astype(np.float32))
    F = oracle.subdots_q3_K_folded(w, rows, k, xq, n)
    for c in range(n):
        qa = q8_1_codes(xq[c])
        for r in range(rows):
            qw = weight_codes(oracle.Q3_K, fields[r])
            sc = np.concatenate([f[1] for f in fields[r]]) - 32
            for b in range(k // 32):
                expect = sum(int(sc[v // 16]) * int(qw[v]) * int(qa[v]) for v in range(32 * b, 32 * b + 32))
                assert F[c, r, b] == expect
