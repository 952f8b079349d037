"""Pins for the oracle's gate/up products fused with SwiGLU (CPU only).

MMQ page, the fusion passage after the MoE dispatch: the gate and up products of one input are
computed together and the GLU is applied at write-back; read as out = silu(g) * u with
silu(g) = g * sigmoid(g).  The products themselves are the oracle's pinned matmul; these tests pin
the combination with forms of silu the oracle does not use (sigmoid through tanh, the odd-part
identity silu(g) - silu(-g) = g, the limits for large |g|), the roles of gate and up, and the
expert form against a loop of dense calls.
"""
import numpy as np
import pytest

import oracle
import synth


def _silu_tanh(g):
    g = np.asarray(g, dtype=np.float64)
    return g * (0.5 + 0.5 * np.tanh(0.5 * g))   # sigmoid(g) = (1 + tanh(g/2)) / 2


def _neg_q8_0(w):
    """Q8_0 blocks with every code negated (codes are in [-127, 127], so exactly)."""
    v = w.copy().reshape(-1, 34)
    q = v[:, 2:].view(np.int8)
    v[:, 2:] = (-q.astype(np.int16)).astype(np.int8).view(np.uint8)
    return v.reshape(w.shape)


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K, oracle.Q8_0])
def test_glu_is_silu_of_gate_times_up(qtype):
    rng = np.random.default_rng(70 + qtype)
    rows, k, n = 9, 512, 4
    wg = synth.gen_weights(qtype, rows, k, rng)
    wu = synth.gen_weights(qtype, rows, k, rng)
    x = (0.05 * rng.standard_normal((n, k))).astype(np.float32)
    y = oracle.matmul_glu(qtype, wg, wu, rows, k, x)
    G = oracle.matmul(qtype, wg, rows, k, x).astype(np.float64)
    U = oracle.matmul(qtype, wu, rows, k, x).astype(np.float64)
    # the gates span silu's curved range, both signs
    assert np.sum((G > 0.25) & (G < 6)) >= 3 and np.sum((G < -0.25) & (G > -6)) >= 3
    ref = _silu_tanh(G) * U
    # one fp32 rounding of the fp64 value (the tanh form cancels for g << 0: absolute 1e-15*|g*u|)
    assert np.all(np.abs(y - ref) <= 1.2e-7 * np.abs(ref) + 1e-15 * np.abs(G * U) + 1e-38)
    # gate and up are not interchangeable: the swapped reading differs on these inputs
    assert not np.allclose(y, _silu_tanh(U) * G, rtol=1e-3)


def test_glu_odd_part_identity():
    """silu(g) - silu(-g) = g: negating the gate weights (exact for Q8_0) gives y1 - y2 = g * u."""
    rng = np.random.default_rng(81)
    rows, k, n = 6, 256, 3
    wg = synth.gen_weights(oracle.Q8_0, rows, k, rng)
    wu = synth.gen_weights(oracle.Q8_0, rows, k, rng)
    x = rng.standard_normal((n, k)).astype(np.float32)
    y1 = oracle.matmul_glu(oracle.Q8_0, wg, wu, rows, k, x).astype(np.float64)
    y2 = oracle.matmul_glu(oracle.Q8_0, _neg_q8_0(wg), wu, rows, k, x).astype(np.float64)
    G = oracle.matmul(oracle.Q8_0, wg, rows, k, x).astype(np.float64)
    assert np.array_equal(oracle.matmul(oracle.Q8_0, _neg_q8_0(wg), rows, k, x).astype(np.float64), -G)
    U = oracle.matmul(oracle.Q8_0, wu, rows, k, x).astype(np.float64)
    scale = np.abs(G * U) + np.abs(y1) + np.abs(y2)
    assert np.all(np.abs((y1 - y2) - G * U) <= 4e-7 * scale)


def test_glu_limits_and_zero():
    """silu(g) -> g for g >> 0, -> 0 for g << 0, silu(0) = 0 (all-zero gate weights)."""
    rng = np.random.default_rng(82)
    rows, k = 4, 256
    wu = synth.gen_weights(oracle.Q8_0, rows, k, rng)
    x = np.ones((2, k), dtype=np.float32)
    x[1] = -1.0
    # gate rows: every code 127 with a large scale -> |g| in the thousands, sign of the column
    wg = np.zeros((rows, (k // 32) * 34), dtype=np.uint8).reshape(-1, 34)
    wg[:, 0:2] = np.frombuffer(np.float16(2.0).tobytes(), dtype=np.uint8)
    wg[:, 2:] = np.uint8(127)
    wg = wg.reshape(rows, -1)
    y = oracle.matmul_glu(oracle.Q8_0, wg, wu, rows, k, x).astype(np.float64)
    G = oracle.matmul(oracle.Q8_0, wg, rows, k, x).astype(np.float64)
    U = oracle.matmul(oracle.Q8_0, wu, rows, k, x).astype(np.float64)
    assert np.all(G[0] > 1000) and np.all(G[1] < -1000)
    assert np.allclose(y[0], G[0] * U[0], rtol=1e-7)
    assert np.all(np.abs(y[1]) <= 1e-300 + 1e-30 * np.abs(G[1] * U[1]))
    zero = np.zeros_like(wg)
    assert np.all(oracle.matmul_glu(oracle.Q8_0, zero, wu, rows, k, x) == 0)


def test_glu_id_is_loop_of_dense():
    rng = np.random.default_rng(83)
    n_exp, rows, k, n_tok, top_k = 4, 10, 256, 6, 2
    wg = synth.gen_weights(oracle.Q4_K, n_exp * rows, k, rng)
    wu = synth.gen_weights(oracle.Q4_K, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok, k)).astype(np.float32)
    ids = rng.integers(0, n_exp, (n_tok, top_k)).astype(np.int32)
    ids[3, 1] = n_exp
    y, bad = oracle.matmul_id_glu(oracle.Q4_K, wg, wu, n_exp, rows, k, x, ids)
    assert bad == 1
    rb = oracle.row_bytes(oracle.Q4_K, k)
    wgm, wum = wg.reshape(n_exp, rows * rb), wu.reshape(n_exp, rows * rb)
    for t in range(n_tok):
        for s in range(top_k):
            e = ids[t, s]
            if not 0 <= e < n_exp:
                assert np.all(np.isnan(y[t, s]))
                continue
            ref = oracle.matmul_glu(oracle.Q4_K, wgm[e], wum[e], rows, k, x[t][None, :])[0]
            assert np.array_equal(y[t, s], ref)
