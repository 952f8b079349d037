"""GPU parity for Q3_K and IQ4_XS (the GP100 patch page, "How" step 3: Q3_K's 3-bit codes carry a
-4 offset, IQ4_XS maps 4-bit indices through a codebook; both have 6-bit scales minus 32).  They
run on the dot4 matrix-vector kernel (one to three columns, activations quantized in the kernel),
the register-streamed matrix-vector kernel (any column count up to 8, any 2-byte aligned rows) and
the tiled kernel (Q3_K parked like Q6_K as scale-folded planes, IQ4_XS like Q8_0 as int8 codes
plus a scale per 32 values), dense, expert-indexed and gate/up-fused.  Bars as everywhere: integer dots from the
production kernels bit-exact, fp32 outputs within gpu_util.assert_close's normalised bound.
"""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, assert_close, col_norms, row_norms, to_dev
from test_gpu_glu import _assert_glu

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q3_K, qmm.IQ4_XS]
TNAME = {qmm.Q3_K: "q3_K", qmm.IQ4_XS: "iq4_xs"}


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


def _folded(qtype, w, rows, k, xq, n):
    if qtype == qmm.Q3_K:
        return oracle.subdots_q3_K_folded(w, rows, k, xq, n)
    return oracle.subdots(qtype, w, rows, k, xq, n)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 5, 8])
@pytest.mark.parametrize("spw", [1, 2, 4])
def test_subdots_matvec_bit_exact(qtype, n, spw):
    """Integer dots of the register-streamed kernel (Q3_K per 16 values, IQ4_XS per 32) at every
    steps-per-wave setting; 40 rows (ragged last row group), 1792 values = 7 steps (odd: rows are
    only 2-byte aligned for Q3_K)."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 1)
    qmm.set_override(qmm.OVR_MV_STEPS, spw)
    rows, k = 40, 1792
    w, x = _case(qtype, rows, k, n, 2000 + n)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_MATVEC).cpu().numpy()
    exp = oracle.subdots(qtype, w, rows, k, xq, n)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3])
def test_subdots_dot4_bit_exact(qtype, n):
    """Integer dots of the dot4 kernel (Q3_K per 16 values over the codes minus 4, IQ4_XS per 32
    over the codebook values): 40 rows, 7 steps, rows 2-byte aligned for Q3_K."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    rows, k = 40, 1792
    w, x = _case(qtype, rows, k, n, 2050 + n)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_MATVEC).cpu().numpy()
    exp = oracle.subdots(qtype, w, rows, k, xq, n)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3])
def test_dot4_fp32_and_q8_1_inputs(qtype, n):
    """The dot4 kernel from fp32 activations (quantized in the kernel) and from q8_1 blocks, on
    ragged rows with K = 7 steps: every output within the bound, and both inputs give the same
    outputs bit for bit (the in-kernel quantization writes the same codes)."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 3)
    rows, k = 333, 1792
    w, x = _case(qtype, rows, k, n, 2060 + n)
    wd, xd = to_dev(w), to_dev(x)
    assert qmm.matvec_kernel(qtype, wd, rows, k, xd, n) == (3, True)
    y = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} dot4 n={n}")
    yq = qmm.matmul_q8_1(wd, qtype, rows, k, to_dev(xq), n).cpu().numpy()
    assert np.array_equal(y, yq)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("J,sk", [(32, 1), (64, 2), (128, 2), (128, 1)])
def test_subdots_tiled_bit_exact(qtype, J, sk):
    """The tiled kernel's integer dots (Q3_K: the scale-folded sc0*D0 + sc1*D1 its planes give)
    at every tile width, stream-K on (units split tiles) and off."""
    qmm.set_override(qmm.OVR_TILE_J, J)
    qmm.set_override(qmm.OVR_STREAMK, sk)
    rows, k, n = 300, 1792, 70
    w, x = _case(qtype, rows, k, n, 2100 + J + sk)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_TILED).cpu().numpy()
    assert np.array_equal(got, _folded(qtype, w, rows, k, xq, n))


def test_subdots_extreme_codes():
    """Codes and scales at the ends of their ranges: Q3_K stored code 0 (value -4) with scale 0
    (value -32) gives v = 128, the one product outside int8 that the hi/lo split must carry;
    IQ4_XS index 0 (-127) with scale 63 (+31)."""
    rows, k, n = 64, 512, 40
    x = np.where(np.arange(n * k).reshape(n, k) % 3 == 0, -1.0, 1.0).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    w3 = np.zeros((rows, k // 256 * 110), dtype=np.uint8)
    w3.reshape(rows, -1, 110)[:, :, 108:110] = np.array([0x00, 0x3C], dtype=np.uint8)   # d = 1
    wi = np.zeros((rows, k // 256 * 136), dtype=np.uint8)
    blk = wi.reshape(rows, -1, 136)
    blk[:, :, 0:2] = np.array([0x00, 0x3C], dtype=np.uint8)
    blk[:, :, 2:4] = 0xFF
    blk[:, :, 4:8] = 0xFF
    for qtype, w in ((qmm.Q3_K, w3), (qmm.IQ4_XS, wi)):
        # matrix-vector: 8 columns (register-streamed) and 3 (dot4); tiled: all 40
        for path, nn in ((qmm.PATH_MATVEC, 8), (qmm.PATH_MATVEC, 3), (qmm.PATH_TILED, n)):
            got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq[:nn]), nn, path).cpu().numpy()
            exp = (oracle.subdots(qtype, w, rows, k, xq[:nn], nn) if path == qmm.PATH_MATVEC
                   else _folded(qtype, w, rows, k, xq[:nn], nn))
            assert np.array_equal(got, exp), (qtype, path, nn)


def _full_check(qtype, rows, k, n, seed, what):
    w, x = _case(qtype, rows, k, n, seed)
    y = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    return assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=what)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 9, 16, 17, 33, 130])
def test_dense_ragged(qtype, n):
    _full_check(qtype, 300, 768, n, 2200 + n, f"{TNAME[qtype]} 300x768 n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_matvec_full_size(qtype, n):
    _full_check(qtype, 4096, 4096, n, 2300 + n, f"{TNAME[qtype]} 4096^2 n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_prefill_full_size_whole_rows(qtype):
    """An FFN up projection at full size, 14336 x 4096 x 512 tokens (stream-K plan), on 256 whole
    output rows (every column of each) plus the first and the last."""
    rows, k, n = 14336, 4096, 512
    w, x = _case(qtype, rows, k, n, 2400)
    y = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    rng = np.random.default_rng(2401)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 256, replace=False)]))
    rb = oracle.row_bytes(qtype, k)
    wsub = np.ascontiguousarray(w.reshape(rows, rb)[sel])
    ref = oracle.matmul_q8_1(qtype, wsub, len(sel), k, xq, n)
    assert_close(np.ascontiguousarray(y[:, sel]), ref, row_norms(qtype, wsub, len(sel), k), col_norms(xq, n, k))


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_moe_small_and_tiled_experts(qtype):
    """Expert-indexed product with both regimes: skewed routing gives experts with <= 8 columns
    (matrix-vector kernel in expert mode) and experts with many (tiled expert kernel); per-slot
    activations; every output against the oracle."""
    n_exp, rows, k, n_tok, top_k = 8, 160, 1024, 120, 2
    g = synth.rngs(2500 + qtype, 3)
    w = synth.gen_weights(qtype, n_exp * rows, k, g[0])
    x = synth.gen_activations(n_tok * top_k, k, g[1])
    ids = synth.gen_routing(n_tok, top_k, n_exp, 1.5, g[2])
    counts = np.bincount(ids.reshape(-1), minlength=n_exp)
    assert counts.min() <= 8 < counts.max()
    y, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=top_k)
    assert qmm.matmul_id_invalid_count(ws) == 0
    y = y.cpu().numpy()
    ref, bad = oracle.matmul_id(qtype, w, n_exp, rows, k, x, top_k, ids)
    assert bad == 0
    xq = oracle.quantize_q8_1(x)
    wn_all = row_norms(qtype, w, n_exp * rows, k).reshape(n_exp, rows)
    xn_all = col_norms(xq, n_tok * top_k, k)
    for t in range(n_tok):
        for s in range(top_k):
            a = t * top_k + s
            assert_close(y[t, s][None], ref[t, s][None], wn_all[ids[t, s]], xn_all[a:a + 1], what=f"pair {t},{s}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 5, 9, 130])
def test_glu_dense(qtype, n):
    """Gate/up fused with SwiGLU: the register-streamed kernel's fused form up to 8 columns, the
    tiled GLU kernel beyond; 200 rows, small activations (gates in silu's curved range); the
    tolerance of the other types' GLU tests (derived there from the product bar)."""
    rows, k = 200, 768
    g = synth.rngs(2600 + n, 3)
    wg = synth.gen_weights(qtype, rows, k, g[0])
    wu = synth.gen_weights(qtype, rows, k, g[1])
    x = (0.05 * synth.gen_activations(n, k, g[2])).astype(np.float32)
    y = qmm.matmul_glu(to_dev(wg), to_dev(wu), qtype, rows, k, to_dev(x)).cpu().numpy()
    yref = oracle.matmul_glu(qtype, wg, wu, rows, k, x)
    G = oracle.matmul(qtype, wg, rows, k, x)
    U = oracle.matmul(qtype, wu, rows, k, x)
    xn = col_norms(oracle.quantize_q8_1(x), n, k)
    _assert_glu(y, yref, G, U, row_norms(qtype, wg, rows, k), row_norms(qtype, wu, rows, k), xn, f"{TNAME[qtype]} n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_modes_without_these_types_refuse(qtype):
    """The fp16-activation mode and the panel layout serve the five other types only."""
    w = to_dev(synth.gen_weights(qtype, 16, 256, synth.rngs(3, 1)[0]))
    x = torch.zeros((1, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(qmm.QmmError) as e:
        qmm.matmul_f16act(w, qtype, 16, 256, x)
    assert e.value.status == -2   # QMM_ERR_TYPE
    assert qmm.repack_bytes(qtype, 16, 256) == 0
    with pytest.raises(qmm.QmmError) as e:
        qmm.repack(w, qtype, 16, 256)
    assert e.value.status == -2
    qmm.set_override(qmm.OVR_MV_KERNEL, 2)        # the LDS-staged kernel cannot serve them
    with pytest.raises(qmm.QmmError):
        qmm.matmul(w, qtype, 16, 256, x)
        torch.cuda.synchronize()
