"""Small and degenerate shapes through every matrix-vector kernel and mode: one to three 256-value
steps (one-, two- and three-wave workgroups), one and seventeen rows (a single ragged row group),
every column count a kernel serves, the fp16-activation mode down to one 32-value block, the
panel layout at one panel per row group, the fused gate/up form; the tiled kernel at one or two
steps, one or 129 rows, every tile width, stream-K on and off; experts at one step.  Every output
against the oracle within the normalised bound (the MMQ page, "shape criteria": n <= 8 runs the
matrix-vector regime at any K, more columns the tiled one)."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, assert_close, col_norms, row_norms, to_dev
from test_gpu_glu import _check_dense as _check_glu

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0, qmm.Q3_K, qmm.IQ4_XS]
TNAME = {qmm.Q4_K: "q4_K", qmm.Q5_K: "q5_K", qmm.Q6_K: "q6_K", qmm.Q8_0: "q8_0", qmm.Q4_0: "q4_0",
         qmm.Q3_K: "q3_K", qmm.IQ4_XS: "iq4_xs"}
# kernels that serve a type at K a multiple of 256 with aligned rows (Q6_K's LDS-staged form needs
# 16-byte aligned rows: K a multiple of 2048)
SERVES = {1: set(TYPES), 2: {qmm.Q4_K, qmm.Q5_K, qmm.Q8_0, qmm.Q4_0, qmm.Q6_K},
          3: {qmm.Q4_K, qmm.Q5_K, qmm.Q8_0, qmm.Q4_0, qmm.Q3_K, qmm.IQ4_XS}}


_KEYS = (qmm.OVR_PATH, qmm.OVR_STREAMK, qmm.OVR_TILE_J, qmm.OVR_MV_KERNEL)


@pytest.fixture(autouse=True)
def _clean_overrides():
    for key in _KEYS:
        qmm.set_override(key, 0)
    yield
    for key in _KEYS:
        qmm.set_override(key, 0)


def _case(qtype, rows, k, n, seed):
    g_w, g_x = synth.rngs(seed, 2)
    return synth.gen_weights(qtype, rows, k, g_w), synth.gen_activations(n, k, g_x)


def _check(qtype, rows, k, n, seed, what):
    w, x = _case(qtype, rows, k, n, seed)
    y = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=what)


@pytest.mark.parametrize("kernel", [1, 2, 3], ids=["regs", "lds", "dot4"])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_every_kernel_few_steps_every_column_count(qtype, kernel):
    if qtype not in SERVES[kernel]:
        pytest.skip("this kernel does not serve the type")
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    ks = (2048,) if kernel == 2 and qtype == qmm.Q6_K else (256, 512, 768)
    ns = range(1, 4) if kernel == 3 else range(1, 9)
    for k in ks:
        for rows in (1, 17):
            for n in ns:
                _check(qtype, rows, k, n, 3000 + 7 * k + 3 * rows + n,
                       f"{TNAME[qtype]} kernel={kernel} {rows}x{k} n={n}")


@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0], ids=TNAME.get)
def test_f16act_few_blocks(qtype):
    """The fp16-activation mode on K below one 64-block chunk: 256 values (8 blocks), and one
    32-value block for the 32-value types."""
    ks = (32, 256) if qtype in (qmm.Q8_0, qmm.Q4_0) else (256,)
    for k in ks:
        for rows, n in ((1, 1), (17, 8)):
            g_w, g_x = synth.rngs(3100 + k + n, 2)
            w = synth.gen_weights(qtype, rows, k, g_w)
            x = synth.gen_activations(n, k, g_x)
            y = qmm.matmul_f16act(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
            ref = oracle.matmul_f16act(qtype, w, rows, k, x)
            xn = np.linalg.norm(x.astype(np.float64), axis=1)
            assert_close(y, ref, row_norms(qtype, w, rows, k), xn, what=f"{TNAME[qtype]} f16act {rows}x{k} n={n}")


@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0], ids=TNAME.get)
def test_packed_one_row(qtype):
    """Panel layout with a single live row (15 zero padding rows) at one and three steps."""
    for k in (256, 768):
        for n in (1, 8, 9):
            w, x = _case(qtype, 1, k, n, 3200 + k + n)
            wd = to_dev(w)
            wp = qmm.repack(wd, qtype, 1, k)
            y = qmm.matmul_packed(wp, qtype, 1, k, to_dev(x)).cpu().numpy()
            xq = oracle.quantize_q8_1(x)
            ref = oracle.matmul_q8_1(qtype, w, 1, k, xq, n)
            assert_close(y, ref, row_norms(qtype, w, 1, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} packed 1x{k} n={n}")


@pytest.mark.parametrize("kernel", [1, 2, 3], ids=["regs", "lds", "dot4"])
@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q8_0, qmm.Q3_K], ids=TNAME.get)
def test_glu_one_step(qtype, kernel):
    """Gate/up fusion at K = 256 and 9 outputs (one full and one ragged group of 8)."""
    if qtype not in SERVES[kernel]:
        pytest.skip("this kernel does not serve the type")
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    for n in ((1, 2, 3) if kernel == 3 else (1, 5, 8)):
        _check_glu(qtype, 9, 256, n, 3300 + n, f"{TNAME[qtype]} glu kernel={kernel} n={n}")


@pytest.mark.parametrize("J", [32, 64, 128])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_tiled_few_steps_and_rows(qtype, J):
    """The tiled kernel on one to two 256-value steps (Q8_0 / Q4_0 also a ragged 288), one and
    129 rows (a single ragged row tile, and one full tile plus one row), 9 to 130 columns, with
    stream-K forced on and off."""
    qmm.set_override(qmm.OVR_PATH, 2)
    qmm.set_override(qmm.OVR_TILE_J, J)
    ks = (256, 512, 288) if qtype in (qmm.Q8_0, qmm.Q4_0) else (256, 512)
    for k in ks:
        for rows in (1, 129):
            for n, sk in ((9, 1), (33, 2), (130, 2)):
                qmm.set_override(qmm.OVR_STREAMK, sk)
                _check(qtype, rows, k, n, 3400 + k + rows + n, f"{TNAME[qtype]} tiled J={J} {rows}x{k} n={n} sk={sk}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_experts_one_step(qtype):
    """Expert-indexed product at K = 256: three experts, one with 40 columns (tiled), one with 3
    (matrix-vector), one with none; 17 rows; top-1 routing."""
    rng = np.random.default_rng(3500 + qtype)
    n_exp, rows, k, n_tok, top_k = 3, 17, 256, 43, 1
    ids = np.zeros((n_tok, top_k), dtype=np.int32)
    ids[:40, 0] = 0
    ids[40:, 0] = 2
    w = synth.gen_weights(qtype, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok, k)).astype(np.float32)
    y, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=1)
    assert qmm.matmul_id_invalid_count(ws) == 0
    y = y.cpu().numpy()
    ref, bad = oracle.matmul_id(qtype, w, n_exp, rows, k, x, 1, ids)
    assert bad == 0
    xq = oracle.quantize_q8_1(x)
    wn = row_norms(qtype, w, n_exp * rows, k).reshape(n_exp, rows)
    xn = col_norms(xq, n_tok, k)
    for t in range(n_tok):
        assert_close(y[t, 0][None], ref[t, 0][None], wn[ids[t, 0]], xn[t:t + 1], what=f"{TNAME[qtype]} token {t}")
