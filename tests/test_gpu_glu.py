"""GPU parity of the gate/up products fused with SwiGLU (the MMQ page's fusion passage), through
the C ABI, against the oracle's matmul_glu / matmul_id_glu on the same seeded inputs.

Tolerance, derived from the product bar: each product is within d = 1e-4 * ||w_r|| * ||x_n|| of
the oracle's (dg for the gate row, du for the up row), and silu has slope at most 1.0998, so
    |y_gpu - y_ref| <= 1.1 * dg * (|U| + du) + |silu(G)| * du + 1e-6 * |y_ref|
with G, U the oracle's products; the last term covers the kernel's fp32 silu (exp, divide,
multiply: a few ulp).
"""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, col_norms, row_norms, to_dev

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0]
TNAME = {qmm.Q4_K: "q4_K", qmm.Q5_K: "q5_K", qmm.Q6_K: "q6_K", qmm.Q8_0: "q8_0", qmm.Q4_0: "q4_0"}


@pytest.fixture(autouse=True)
def _clean_overrides():
    keys = (qmm.OVR_PATH, qmm.OVR_TILE_J, qmm.OVR_MV_KERNEL)
    for key in keys:
        qmm.set_override(key, 0)
    yield
    for key in keys:
        qmm.set_override(key, 0)


def _silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def _glu_bound(G, U, wgn, wun, xn):
    dg = 1e-4 * np.outer(xn, wgn)
    du = 1e-4 * np.outer(xn, wun)
    G = G.astype(np.float64)
    U = U.astype(np.float64)
    return 1.1 * dg * (np.abs(U) + du) + np.abs(_silu(G)) * du + 1e-6 * np.abs(_silu(G) * U) + 1e-30


def _assert_glu(y, yref, G, U, wgn, wun, xn, what):
    assert y.shape == yref.shape
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y.astype(np.float64) - yref.astype(np.float64))
    bound = _glu_bound(G, U, wgn, wun, xn)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), f"{what}: error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"


def _inputs(qtype, rows, k, n, seed, scale=0.05):
    g = synth.rngs(seed, 3)
    wg = synth.gen_weights(qtype, rows, k, g[0])
    wu = synth.gen_weights(qtype, rows, k, g[1])
    # small activations put many gates in silu's curved range (|g| of order 1)
    x = (scale * synth.gen_activations(n, k, g[2])).astype(np.float32)
    return wg, wu, x


def _check_dense(qtype, rows, k, n, seed, what):
    wg, wu, x = _inputs(qtype, rows, k, n, seed)
    y = qmm.matmul_glu(to_dev(wg), to_dev(wu), qtype, rows, k, to_dev(x)).cpu().numpy()
    yref = oracle.matmul_glu(qtype, wg, wu, rows, k, x)
    G = oracle.matmul(qtype, wg, rows, k, x)
    U = oracle.matmul(qtype, wu, rows, k, x)
    xn = col_norms(oracle.quantize_q8_1(x), n, k)
    _assert_glu(y, yref, G, U, row_norms(qtype, wg, rows, k), row_norms(qtype, wu, rows, k), xn, what)
    return G


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 3, 8, 9, 40, 130])
def test_glu_dense(qtype, n):
    # 200 rows: three 64-output tiles and a ragged one, 25 matrix-vector workgroups of 8;
    # Q8_0 at k = 544 ends in a partial 256-value step
    k = 544 if qtype in (qmm.Q8_0, qmm.Q4_0) else 512
    G = _check_dense(qtype, 200, k, n, 900 + n, f"{TNAME[qtype]} n={n}")
    assert np.mean(np.abs(G) < 4) > 0.2    # the gates exercise silu's curve, not only its limits


@pytest.mark.parametrize("J", [32, 64, 128])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_glu_dense_tile_widths(qtype, J):
    qmm.set_override(qmm.OVR_TILE_J, J)
    _check_dense(qtype, 300, 1024, 150, 950 + J, f"{TNAME[qtype]} J={J}")


@pytest.mark.parametrize("kernel", [0, 1, 2, 3], ids=["auto", "regs", "lds", "dot4"])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_glu_matvec_kernels(qtype, n, kernel):
    """Each matrix-vector kernel's fused form (a forced kernel that cannot serve the call falls
    back to the register-streamed one): 232 rows = 29 workgroups of 8 outputs, the last ragged."""
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    _check_dense(qtype, 229, 1024, n, 1200 + 10 * n + kernel, f"{TNAME[qtype]} n={n} kernel={kernel}")


@pytest.mark.parametrize("kernel", [1, 2], ids=["regs", "lds"])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 8])
def test_glu_matvec_several_steps_per_wave(qtype, n, kernel):
    """More steps than waves (17; Q6_K 24, whose rows must stay 16-byte aligned for the LDS-staged
    kernel): some waves compute a step while the next step's loads are in flight."""
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    k = 6144 if qtype == qmm.Q6_K else 4352
    _check_dense(qtype, 45, k, n, 1280 + 10 * n + kernel, f"{TNAME[qtype]} k={k} n={n} kernel={kernel}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 5, 8])
def test_glu_single_step_k(qtype, n):
    """K = 256 (one wave per matrix-vector workgroup): gate and up sums of every column."""
    _check_dense(qtype, 100, 256, n, 1260 + n, f"{TNAME[qtype]} k=256 n={n}")


def test_glu_dense_tiled_path_for_few_columns():
    qmm.set_override(qmm.OVR_PATH, 2)
    _check_dense(qmm.Q4_K, 136, 768, 5, 990, "q4_K n=5 tiled")


@pytest.mark.parametrize("kernel", [0, 1], ids=["auto", "regs"])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_glu_expert(qtype, kernel):
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)   # the small experts' matrix-vector kernel
    n_exp, rows, k, n_tok, top_k = 10, 136, 512, 150, 2
    g = synth.rngs(1000 + qtype, 4)
    wg = synth.gen_weights(qtype, n_exp * rows, k, g[0])
    wu = synth.gen_weights(qtype, n_exp * rows, k, g[1])
    x = (0.05 * synth.gen_activations(n_tok, k, g[2])).astype(np.float32)
    ids = synth.gen_routing(n_tok, top_k, n_exp, 1.5, g[3])
    ids[5, 1] = n_exp       # invalid ids: skipped, counted, rows left untouched
    ids[77, 0] = -3
    sentinel = -12345.0
    out = torch.full((n_tok, top_k, rows), sentinel, dtype=torch.float32, device=DEV)
    y, ws = qmm.matmul_id_glu(to_dev(wg), to_dev(wu), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), out=out)
    assert qmm.matmul_id_invalid_count(ws) == 2
    y = y.cpu().numpy()
    yref, bad = oracle.matmul_id_glu(qtype, wg, wu, n_exp, rows, k, x, ids, fill=sentinel)
    assert bad == 2
    assert np.all(y[5, 1] == sentinel) and np.all(y[77, 0] == sentinel)
    counts = np.bincount(ids[(ids >= 0) & (ids < n_exp)], minlength=n_exp)
    assert counts.min() <= 8 < counts.max()   # both the matrix-vector and the tiled experts
    Gf, _ = oracle.matmul_id(qtype, wg, n_exp, rows, k, x, 1, ids)
    Uf, _ = oracle.matmul_id(qtype, wu, n_exp, rows, k, x, 1, ids)
    xn_tok = col_norms(oracle.quantize_q8_1(x), n_tok, k)
    rbg = row_norms(qtype, wg, n_exp * rows, k).reshape(n_exp, rows)
    rbu = row_norms(qtype, wu, n_exp * rows, k).reshape(n_exp, rows)
    for t in range(n_tok):
        for s in range(top_k):
            e = ids[t, s]
            if not 0 <= e < n_exp:
                continue
            _assert_glu(y[t, s][None], yref[t, s][None], Gf[t, s][None], Uf[t, s][None], rbg[e], rbu[e],
                        xn_tok[t:t + 1], f"{TNAME[qtype]} token {t} slot {s} expert {e}")


def test_glu_matches_unfused_products():
    """The fused call against silu(.)*(.) of two unfused library calls on the same input."""
    qtype, rows, k, n = qmm.Q4_K, 264, 2048, 77
    wg, wu, x = _inputs(qtype, rows, k, n, 1111)
    dg, du, dx = to_dev(wg), to_dev(wu), to_dev(x)
    y = qmm.matmul_glu(dg, du, qtype, rows, k, dx).cpu().numpy().astype(np.float64)
    G = qmm.matmul(dg, qtype, rows, k, dx).cpu().numpy()
    U = qmm.matmul(du, qtype, rows, k, dx).cpu().numpy()
    xn = col_norms(oracle.quantize_q8_1(x), n, k)
    wgn, wun = row_norms(qtype, wg, rows, k), row_norms(qtype, wu, rows, k)
    # both sides within the product bar of the oracle: twice the bound
    assert np.all(np.abs(y - _silu(G) * U) <= 2 * _glu_bound(G, U, wgn, wun, xn))
