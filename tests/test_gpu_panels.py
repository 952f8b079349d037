"""GPU parity of the panel layout (the one-time weight repack, after the "QTensor and QMatMul"
page's section on the 8-column Q4K repack): the repack kernel's bytes against the oracle's repack,
bit-exact; the products that read panels against the oracle's product on the ORIGINAL blocks, to
the same normalised bound as every other fp32 output (gpu_util.assert_close).
"""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import assert_close, col_norms, row_norms, to_dev

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0]
TNAME = {qmm.Q4_K: "q4_K", qmm.Q5_K: "q5_K", qmm.Q6_K: "q6_K", qmm.Q8_0: "q8_0", qmm.Q4_0: "q4_0"}


def _reset_overrides():
    for key in (qmm.OVR_PATH, qmm.OVR_STREAMK, qmm.OVR_TILE_J, qmm.OVR_MV_STEPS, qmm.OVR_MV_KERNEL, qmm.OVR_FUSE_COLS):
        qmm.set_override(key, 0)


@pytest.fixture(autouse=True)
def _clean_overrides():
    _reset_overrides()
    yield
    _reset_overrides()


def _case(qtype, rows, k, n, seed):
    g_w, g_x = synth.rngs(seed, 2)
    return synth.gen_weights(qtype, rows, k, g_w), synth.gen_activations(n, k, g_x)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("rows,k", [(1, 256), (37, 768), (300, 4096), (4096, 4096)])
def test_repack_bytes_match_oracle(qtype, rows, k):
    w = synth.gen_weights(qtype, rows, k, synth.rngs(900 + rows, 1)[0])
    assert qmm.repack_bytes(qtype, rows, k) == oracle.panel_bytes(qtype, rows, k)
    got = qmm.repack(to_dev(w), qtype, rows, k).cpu().numpy()
    exp = oracle.repack_panels(qtype, w, rows, k)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp), np.flatnonzero(got != exp)[:8]


def _check_packed(qtype, rows, k, n, seed, what):
    w, x = _case(qtype, rows, k, n, seed)
    wp = qmm.repack(to_dev(w), qtype, rows, k)
    y = qmm.matmul_packed(wp, qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    return assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=what)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 9, 17, 33, 130])
def test_packed_dense_ragged(qtype, n):
    """300 rows (19 row groups, the last with 12 live rows; 3 row tiles, the last ragged), k = 768
    (3 steps): the matrix-vector kernel up to 8 columns, the tiled kernel beyond."""
    _check_packed(qtype, 300, 768, n, 950 + n, f"{TNAME[qtype]} packed 300x768 n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 5, 8])
def test_packed_single_step_k(qtype, n):
    """K = 256: one panel per row group, one wave per matrix-vector workgroup."""
    _check_packed(qtype, 77, 256, n, 960 + n, f"{TNAME[qtype]} packed 77x256 n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 8])
def test_packed_matvec_full_size(qtype, n):
    _check_packed(qtype, 4096, 4096, n, 970 + n, f"{TNAME[qtype]} packed 4096^2 n={n}")



@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("k", [4352, 14336])
@pytest.mark.parametrize("n", [1, 5, 8])
def test_packed_matvec_several_steps_per_wave(qtype, k, n):
    """More than 16 steps (17 and 56): the waves of the matrix-vector kernel take several steps,
    each computed from the panel pieces in its registers while the next step's pieces load."""
    _check_packed(qtype, 40, k, n, 1300 + n + k % 97, f"{TNAME[qtype]} packed k={k} n={n}")

@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_packed_matches_original_layout_bitwise_matvec(qtype):
    """Same kernel, same arithmetic: the LDS-staged kernel reading panels gives exactly the bits it
    gives on the original blocks."""
    rows, k = 1000, 2048
    w, x = _case(qtype, rows, k, 5, 990)
    wd, xd = to_dev(w), to_dev(x)
    qmm.set_override(qmm.OVR_MV_KERNEL, 2)
    y0 = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
    y1 = qmm.matmul_packed(qmm.repack(wd, qtype, rows, k), qtype, rows, k, xd).cpu().numpy()
    assert np.array_equal(y0, y1)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("J,sk", [(32, 1), (64, 2), (128, 2), (128, 1)])
def test_packed_tiled_matches_original_layout_bitwise(qtype, J, sk):
    """The tiled kernel reading panels against itself on the original blocks, at every tile width,
    stream-K on and off: identical bits."""
    rows, k, n = 520, 1536, 100
    w, x = _case(qtype, rows, k, n, 995 + J)
    wd, xd = to_dev(w), to_dev(x)
    qmm.set_override(qmm.OVR_TILE_J, J)
    qmm.set_override(qmm.OVR_STREAMK, sk)
    y0 = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
    y1 = qmm.matmul_packed(qmm.repack(wd, qtype, rows, k), qtype, rows, k, xd).cpu().numpy()
    assert np.array_equal(y0, y1)
    xq = oracle.quantize_q8_1(x)
    assert_close(y1, oracle.matmul_q8_1(qtype, w, rows, k, xq, n), row_norms(qtype, w, rows, k), col_norms(xq, n, k))


@pytest.mark.parametrize("case", synth.PREFILL_CASES, ids=lambda c: c["name"])
def test_packed_prefill_whole_rows(case):
    """The prefill projections at full size from panels: 256 whole output rows against the oracle."""
    w, x = synth.make_dense(case)
    qtype, rows, k, n = case["qtype"], case["rows"], case["k"], case["n"]
    wp = qmm.repack(to_dev(w), qtype, rows, k)
    y = qmm.matmul_packed(wp, qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    rng = np.random.default_rng(17)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 256, replace=False)]))
    rb = oracle.row_bytes(qtype, k)
    wsub = np.ascontiguousarray(w.reshape(rows, rb)[sel])
    ref = oracle.matmul_q8_1(qtype, wsub, len(sel), k, xq, n)
    assert_close(np.ascontiguousarray(y[:, sel]), ref, row_norms(qtype, wsub, len(sel), k), col_norms(xq, n, k),
                 what=case["name"])


def test_packed_refusals():
    w = to_dev(synth.gen_weights(qmm.Q8_0, 16, 96, synth.rngs(1, 1)[0]))
    with pytest.raises(qmm.QmmError) as e:
        qmm.repack(w, qmm.Q8_0, 16, 96)             # k not a multiple of 256
    assert e.value.status == -3   # QMM_ERR_SHAPE
    assert qmm.repack_bytes(qmm.Q8_0, 16, 96) == 0
    x = torch.zeros((1, 96), dtype=torch.float32, device="cuda:0")
    with pytest.raises(qmm.QmmError) as e:
        qmm.matmul_packed(torch.zeros(4352, dtype=torch.uint8, device="cuda:0"), qmm.Q8_0, 16, 96, x)
    assert e.value.status == -3   # QMM_ERR_SHAPE
    w2 = to_dev(synth.gen_weights(qmm.Q4_K, 16, 256, synth.rngs(2, 1)[0]))
    small = torch.zeros(100, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(qmm.QmmError) as e:
        qmm.repack(w2, qmm.Q4_K, 16, 256, out=small)  # output smaller than the layout
    assert e.value.status == -1   # QMM_ERR_ARG
