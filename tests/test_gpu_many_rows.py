"""Matrix-vector calls with many 16-row groups (thousands of workgroups, several per compute unit
over the call): the dot4 kernel that serves one column from 8192 rows on, forced at one to three
columns, and its fused gate/up form (the MMQ page, "MMVQ vs MMQ" table: decode reads every weight
once).  Every output against the oracle within the normalised bound, ragged row counts, fp32 and
q8_1 inputs, the automatic kernel choice, bitwise reruns, and no output row left unwritten."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, assert_close, col_norms, row_norms, to_dev
from test_gpu_glu import _check_dense as _check_glu

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q4_K, qmm.Q5_K, qmm.Q8_0, qmm.Q4_0]   # the types the dot4 kernel serves
TNAME = {qmm.Q4_K: "q4_K", qmm.Q5_K: "q5_K", qmm.Q8_0: "q8_0", qmm.Q4_0: "q4_0"}
ROWS = 40001   # 2501 row groups of 16, the last one ragged


@pytest.fixture(autouse=True)
def _clean_overrides():
    qmm.set_override(qmm.OVR_MV_KERNEL, 0)
    yield
    qmm.set_override(qmm.OVR_MV_KERNEL, 0)


def _case(qtype, rows, k, n, seed):
    g_w, g_x = synth.rngs(seed, 2)
    return synth.gen_weights(qtype, rows, k, g_w), synth.gen_activations(n, k, g_x)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3])
def test_dot4_many_row_groups_fp32_input(qtype, n):
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    k = 512
    w, x = _case(qtype, ROWS, k, n, 1400 + n)
    wd = to_dev(w)
    xd = to_dev(x)
    assert qmm.matvec_kernel(qtype, wd, ROWS, k, xd, n)[0] == 3
    y = qmm.matmul(wd, qtype, ROWS, k, xd).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, ROWS, k, xq, n)
    assert_close(y, ref, row_norms(qtype, w, ROWS, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} n={n}")
    y2 = qmm.matmul(wd, qtype, ROWS, k, xd).cpu().numpy()
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_dot4_many_row_groups_q8_1_input(qtype):
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    k, n = 768, 3
    w, x = _case(qtype, ROWS, k, n, 1410)
    xq = oracle.quantize_q8_1(x)
    y = qmm.matmul_q8_1(to_dev(w), qtype, ROWS, k, to_dev(xq), n).cpu().numpy()
    ref = oracle.matmul_q8_1(qtype, w, ROWS, k, xq, n)
    assert_close(y, ref, row_norms(qtype, w, ROWS, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} q8_1 input")


@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q8_0], ids=TNAME.get)
def test_automatic_choice_at_many_rows(qtype):
    """One column at 8192 rows and more takes the dot4 kernel by itself; so do three columns at
    12288 rows and more (there in workgroups of 4 waves, each wave streaming 4 of the 16 steps)."""
    for rows, k, n in ((16389, 1024, 1), (16389, 4096, 3)):
        w, x = _case(qtype, rows, k, n, 1420 + n)
        wd, xd = to_dev(w), to_dev(x)
        assert qmm.matvec_kernel(qtype, wd, rows, k, xd, n)[0] == 3
        y = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
        xq = oracle.quantize_q8_1(x)
        ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
        assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} auto n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 3])
def test_dot4_glu_many_row_groups(qtype, n):
    """The fused gate/up form: 8 outputs per row group, 20001 outputs = 2501 groups."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    _check_glu(qtype, 20001, 512, n, 1430 + n, f"{TNAME[qtype]} glu n={n}")


def test_dot4_output_rows_written_once_each():
    """Every output row is written: y starts as NaN, and a row group left out would keep NaNs."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    qtype, k, n = qmm.Q8_0, 256, 2
    w, x = _case(qtype, ROWS, k, n, 1440)
    out = torch.full((n, ROWS), float("nan"), dtype=torch.float32, device=DEV)
    y = qmm.matmul(to_dev(w), qtype, ROWS, k, to_dev(x), out=out).cpu().numpy()
    assert np.all(np.isfinite(y))
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, ROWS, k, xq, n)
    assert_close(y, ref, row_norms(qtype, w, ROWS, k), col_norms(xq, n, k), what="q8_0 nan-filled output")
