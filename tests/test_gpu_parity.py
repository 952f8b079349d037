"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle on identical
seeded inputs.

Bars (both sides take every integer decision in the same precision):
  * q8_1 bytes (codes, fp16 d and s): bit-exact.
  * integer sub-block dots from the production kernels' own accumulators: bit-exact.
  * fp32 outputs: |Y_gpu - Y_oracle| <= 1e-4 * ||w_r|| * ||x_n|| (gpu_util.assert_close).
Full-size prefill and MoE workloads are checked on 256 whole output rows (every column of each),
the oracle running on just those weight rows.
"""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, assert_close, col_norms, row_norms, to_dev

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


# ---------------------------------------------------------------------------------------------
# a1: q8_1 quantization, bit-exact
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n,k", [(1, 32), (3, 256), (17, 4096), (64, 14336), (512, 4096)])
def test_quantize_bit_exact_random(n, k):
    rng = np.random.default_rng(100 + n)
    x = (rng.standard_normal((n, k)) * rng.uniform(1e-3, 1e3, (n, 1))).astype(np.float32)
    got = qmm.quantize_q8_1(to_dev(x)).cpu().numpy()
    exp = oracle.quantize_q8_1(x)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


def test_quantize_bit_exact_special_blocks():
    rows = []
    rows.append(np.zeros(32))                                         # zero block
    t = np.zeros(32); t[:6] = [15.875, 0.3125, -0.3125, 0.0625, -0.0625, 1.5625]
    rows.append(t)                                                    # exact rounding ties
    s = np.zeros(32); s[7] = -3.0
    rows.append(s)                                                    # single spike
    rows.append(np.full(32, 0.7))                                     # constant
    rows.append(np.linspace(-1e-38, 1e-38, 32))                       # fp32-subnormal scale
    rows.append(np.linspace(-6e4, 6.5e4, 32))                         # d near fp16 range
    rows.append(np.array([1e30] + [1.0] * 31))                        # d overflows fp16 -> inf
    d = np.zeros(32); d[:2] = [127.031005859375, 100.51]
    rows.append(d)                                                    # unrounded-divisor case
    x = np.stack(rows).astype(np.float32)
    got = qmm.quantize_q8_1(to_dev(x)).cpu().numpy()
    exp = oracle.quantize_q8_1(x)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


def _near_boundary_rows(rng, nrows):
    """Blocks whose values sit on, just below and just above half-integer multiples of the block
    scale d32 = amax/127 (fp32), where the code depends on the last bit of x/d32."""
    rows = []
    for _ in range(nrows):
        blocks = []
        for _ in range(8):
            amax = np.float32(rng.uniform(0.01, 100.0))
            d32 = np.float32(amax / np.float32(127.0))
            ks = rng.integers(-126, 126, 31)
            x = (ks.astype(np.float32) + np.float32(0.5)) * d32
            step = rng.integers(-2, 3, 31)
            x = np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), np.where(step > 0, np.nextafter(x, np.float32(np.inf)), x))
            x = np.clip(x, -amax, amax).astype(np.float32)
            blocks.append(np.concatenate([[amax if rng.random() < 0.5 else -amax], x]).astype(np.float32))
        rows.append(np.concatenate(blocks))
    return np.stack(rows).astype(np.float32)


def test_quantize_bit_exact_near_rounding_boundaries():
    x = _near_boundary_rows(np.random.default_rng(123), 64)     # 64 rows x 256 values
    got = qmm.quantize_q8_1(to_dev(x)).cpu().numpy()
    exp = oracle.quantize_q8_1(x)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


# ---------------------------------------------------------------------------------------------
# a5: integer sub-block dots from the production kernels, bit-exact
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 5, 8])
def test_subdots_matvec_bit_exact(qtype, n):
    k = 96 if qtype == qmm.Q8_0 else 512          # Q8_0: a ragged last 256-value step
    rows = 40                                      # not a multiple of the 16-row group
    w, x = _case(qtype, rows, k, n, 200 + n)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_MATVEC).cpu().numpy()
    exp = oracle.subdots(qtype, w, rows, k, xq, n)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


def _tiled_subdots_check(qtype, rows, k, n, seed):
    w, x = _case(qtype, rows, k, n, seed)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_TILED).cpu().numpy()
    if qtype == qmm.Q6_K:
        exp = oracle.subdots_q6_K_folded(w, rows, k, xq, n)
    else:
        exp = oracle.subdots(qtype, w, rows, k, xq, n)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [3, 40])
def test_subdots_tiled_bit_exact(qtype, n):
    """The tiled kernel's integer dots from its production instantiation: the tiled activation
    layout written by the relayout pass, the seeded integer accumulator (Q4_K, Q5_K) and the
    scale-folded hi/lo planes (Q6_K); only the epilogue stores the integer instead of folding it."""
    _tiled_subdots_check(qtype, 200, 352 if qtype == qmm.Q8_0 else 512, n, 300 + n)


@pytest.mark.parametrize("J", [32, 64, 128])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_subdots_tiled_stream_k_and_tile_widths(qtype, J):
    """The production plan with stream-K forced on: units start and end inside tiles, so each
    tile's steps come from several units; every tile width."""
    qmm.set_override(qmm.OVR_STREAMK, 2)
    qmm.set_override(qmm.OVR_TILE_J, J)
    rows, k, n = 300, (2080 if qtype == qmm.Q8_0 else 2048), 70
    p = qmm.plan_dense(qtype, rows, k, n)
    assert p["stream_k"] == 1 and p["tile_j"] == J
    _tiled_subdots_check(qtype, rows, k, n, 310 + J)


def test_subdots_tiled_extreme_codes():
    """Integer dots at the edges of the seeded accumulator's range: Q4_K / Q5_K codes all at their
    maximum against q8_1 codes of +-127 (|D| = 32 * 31 * 127 for Q5_K, below 2^22)."""
    rows, k, n = 130, 512, 33
    # one sign per 32-value block, alternating over blocks and columns: every q8_1 code is +-127
    blk = np.arange(k)[None, :] // 32 + np.arange(n)[:, None]
    x = np.where(blk % 2 == 0, 1.0, -1.0).astype(np.float32)
    xq = oracle.quantize_q8_1(x)
    for qtype in (qmm.Q4_K, qmm.Q5_K):
        w = synth.gen_weights(qtype, rows, k, np.random.default_rng(320))
        blocks = w.reshape(rows, k // 256, qmm.BLOCK_BYTES[qtype])
        blocks[:, :, 16:] = 0xFF                      # every low nibble and (Q5_K) fifth bit set
        got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_TILED).cpu().numpy()
        exp = oracle.subdots(qtype, w, rows, k, xq, n)
        assert np.abs(exp).max() == (31 if qtype == qmm.Q5_K else 15) * 32 * 127
        assert np.array_equal(got, exp)


# ---------------------------------------------------------------------------------------------
# fp32 outputs, full comparison at sizes the oracle finishes quickly
# ---------------------------------------------------------------------------------------------
def _full_check(qtype, rows, k, n, seed, what):
    w, x = _case(qtype, rows, k, n, seed)
    y = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    return assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=what)


def test_dense_small_workload():
    """Q4_K 512 x 1024 weight times 16 tokens (the small dense workload)."""
    c = synth.DENSE_SMALL
    w, x = synth.make_dense(c)
    y = qmm.matmul(to_dev(w), c["qtype"], c["rows"], c["k"], to_dev(x)).cpu().numpy()
    assert y.shape == (16, 512)
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(c["qtype"], w, c["rows"], c["k"], xq, c["n"])
    assert_close(y, ref, row_norms(c["qtype"], w, c["rows"], c["k"]), col_norms(xq, c["n"], c["k"]))


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 9, 16, 17, 33, 130])
def test_dense_ragged(qtype, n):
    k = 160 if qtype == qmm.Q8_0 else 768
    _full_check(qtype, 300, k, n, 400 + n, f"{TNAME[qtype]} 300x{k} n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_dense_single_block_k(qtype):
    k = 32 if qtype == qmm.Q8_0 else 256
    for n in (1, 12):
        _full_check(qtype, 129, k, n, 450 + n, f"{TNAME[qtype]} k={k} n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", range(1, 9))
def test_single_step_k_every_column_count(qtype, n):
    """K = 256: the LDS-staged kernel runs one wave per workgroup, so its 128 (row, column) sums
    over the waves fall two to a thread; every column count it serves, every output."""
    _full_check(qtype, 77, 256, n, 1180 + n, f"{TNAME[qtype]} k=256 n={n}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_matvec_workload_full(qtype, n):
    """The matrix-vector workload at full size: 4096 x 4096, every output compared."""
    _full_check(qtype, 4096, 4096, n, 500 + n, f"{TNAME[qtype]} 4096^2 n={n}")


@pytest.mark.parametrize("spw", [1, 2, 4])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_matvec_steps_per_wave(qtype, spw):
    """Every steps-per-wave variant of the matrix-vector kernel, on a K that leaves a partial
    pass (several passes for one step per wave) and ragged rows, against the oracle."""
    qmm.set_override(qmm.OVR_MV_STEPS, spw)
    k = 2080 if qmm.Q8_0 == qtype else 4352
    for n in (1, 6):
        _full_check(qtype, 77, k, n, 470 + spw + n, f"{TNAME[qtype]} spw={spw} n={n}")
    w, x = _case(qtype, 77, k, 5, 480 + spw)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, 77, k, to_dev(xq), 5, qmm.PATH_MATVEC).cpu().numpy()
    assert np.array_equal(got, oracle.subdots(qtype, w, 77, k, xq, 5))


MV_KERNELS = [1, 2, 3]     # register-streamed, LDS-staged MFMA, dot4
MV_KNAME = {1: "regs", 2: "lds", 3: "dot4"}


@pytest.mark.parametrize("kernel", MV_KERNELS, ids=MV_KNAME.get)
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_matvec_kernel_variants(qtype, kernel):
    """Every matrix-vector kernel on shapes it serves (aligned rows, K a multiple of 256): ragged
    rows, more 256-value steps than waves so some waves take two, every column-count class the
    kernel handles; fp32 outputs and the integer sub-block dots."""
    if kernel == 3 and qtype == qmm.Q6_K:
        pytest.skip("the dot4 kernel serves Q4_K, Q5_K, Q8_0 and Q4_0")
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    k = 6144 if qtype == qmm.Q6_K else 4352
    ns = (1, 2, 3) if kernel == 3 else (1, 3, 4, 5, 8)
    for n in ns:
        _full_check(qtype, 77, k, n, 520 + n, f"{TNAME[qtype]} {MV_KNAME[kernel]} n={n}")
    nd = 3 if kernel == 3 else 7
    w, x = _case(qtype, 77, k, nd, 530)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, 77, k, to_dev(xq), nd, qmm.PATH_MATVEC).cpu().numpy()
    assert np.array_equal(got, oracle.subdots(qtype, w, 77, k, xq, nd))



@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 8])
def test_matvec_lds_kernel_many_steps_per_wave(qtype, n):
    """The LDS-staged kernel at K = 14336 (56 steps on 16 waves): every wave computes three or four
    steps, each while the next step's loads are in flight, so a step must not read the registers
    the next step's loads refill; fp32 outputs and the integer sub-block dots."""
    qmm.set_override(qmm.OVR_MV_KERNEL, 2)
    rows, k = 40, 14336
    _full_check(qtype, rows, k, n, 590 + n, f"{TNAME[qtype]} lds k={k} n={n}")
    w, x = _case(qtype, rows, k, n, 595 + n)
    xq = oracle.quantize_q8_1(x)
    got = qmm.debug_subdots(to_dev(w), qtype, rows, k, to_dev(xq), n, qmm.PATH_MATVEC).cpu().numpy()
    assert np.array_equal(got, oracle.subdots(qtype, w, rows, k, xq, n))

def _at_offset(a, off):
    """Device copy of numpy bytes whose data pointer sits `off` bytes past a 256-byte boundary."""
    buf = torch.zeros(a.nbytes + 512, dtype=torch.uint8, device=DEV)
    base = (-buf.data_ptr()) % 256
    view = buf[base + off: base + off + a.nbytes]
    view.copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)))
    assert view.data_ptr() % 256 == off
    return view


@pytest.mark.parametrize("qtype,woff", [(qmm.Q4_K, 16), (qmm.Q5_K, 16), (qmm.Q6_K, 16), (qmm.Q8_0, 4),
                                        (qmm.Q8_0, 36)], ids=["q4_K", "q5_K", "q6_K", "q8_0_w4", "q8_0_w36"])
def test_matvec_lds_kernel_at_minimum_alignment(qtype, woff):
    """The LDS-staged kernel at the least alignment it accepts: q8_1 activations 4 bytes past a
    16-byte boundary (the 36-byte blocks are re-laid at park time), Q8_0 weights 4 bytes off."""
    rows, k = 77, 4352 if qtype != qmm.Q6_K else 6144
    qmm.set_override(qmm.OVR_MV_KERNEL, 2)
    for n in (1, 3, 8):
        w, x = _case(qtype, rows, k, n, 560 + n)
        xq = oracle.quantize_q8_1(x)
        wd, xd = _at_offset(w, woff), _at_offset(xq, 4)
        assert qmm.matvec_kernel(qtype, wd, rows, k, xd, n, x_fp32=False) == (2, False)
        y = qmm.matmul_q8_1(wd, qtype, rows, k, xd, n).cpu().numpy()
        ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
        assert_close(y, ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k), what=f"{TNAME[qtype]} n={n}")
        got = qmm.debug_subdots(wd, qtype, rows, k, xd, n, qmm.PATH_MATVEC).cpu().numpy()
        assert np.array_equal(got, oracle.subdots(qtype, w, rows, k, xq, n))


@pytest.mark.parametrize("kernel,qtype,k,n", [(2, qmm.Q6_K, 768, 1),    # 630-byte rows: not 16-byte aligned
                                              (3, qmm.Q6_K, 4096, 1),   # dot4 serves Q4_K / Q8_0 only
                                              (3, qmm.Q4_K, 4096, 4),   # dot4 takes at most 3 columns
                                              (3, qmm.Q4_0, 2080, 1)])  # Q4_0, K not a multiple of 256
def test_forced_matvec_kernel_refuses_unsupported_call(kernel, qtype, k, n):
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    w, x = _case(qtype, 32, k, n, 540)
    with pytest.raises(qmm.QmmError):
        qmm.matmul(to_dev(w), qtype, 32, k, to_dev(x))
        torch.cuda.synchronize()


FUSED_SHAPES = [(qmm.Q4_K, 1), (qmm.Q4_K, 2), (qmm.Q8_0, 1), (qmm.Q8_0, 2), (qmm.Q8_0, 3),
                (qmm.Q4_K, 3), (qmm.Q4_K, 5), (qmm.Q4_K, 8), (qmm.Q8_0, 4), (qmm.Q8_0, 8),
                (qmm.Q6_K, 1), (qmm.Q6_K, 2), (qmm.Q6_K, 3), (qmm.Q6_K, 8),
                (qmm.Q5_K, 1), (qmm.Q5_K, 2), (qmm.Q5_K, 8)]
# automatic choice and the LDS-staged kernel everywhere; dot4 where it serves (not Q6_K, <= 3 columns)
FUSED_CASES = [(t, n, kern) for kern in (0, 2, 3) for t, n in FUSED_SHAPES if kern != 3 or (t != qmm.Q6_K and n <= 3)]


@pytest.mark.parametrize("qtype,n,kernel", FUSED_CASES,
                         ids=[f"{TNAME[t]}-n{n}-{('auto', '', 'lds', 'dot4')[kern]}" for t, n, kern in FUSED_CASES])
def test_fused_quantize_matches_separate_quantize_bitwise(qtype, n, kernel):
    """fp32 input to the matrix-vector path with fusion forced for every column count: the dot4 or
    LDS-staged kernel quantizes the activations itself; the output equals
    quantize_q8_1 followed by the q8_1-input product bit for bit, and the oracle's.  More 256-value
    steps than waves, so some waves quantize two steps."""
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    qmm.set_override(qmm.OVR_FUSE_COLS, 8)                    # every column count fused here
    k = 6144 if qtype == qmm.Q6_K else 4352
    w, x = _case(qtype, 77, k, n, 560 + n)
    wd, xd = to_dev(w), to_dev(x)
    fused = qmm.matmul(wd, qtype, 77, k, xd)
    separate = qmm.matmul_q8_1(wd, qtype, 77, k, qmm.quantize_q8_1(xd), n)
    assert torch.equal(fused, separate)
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qtype, w, 77, k, xq, n)
    assert_close(fused.cpu().numpy(), ref, row_norms(qtype, w, 77, k), col_norms(xq, n, k))


@pytest.mark.parametrize("qtype,n", [(qmm.Q4_K, 2), (qmm.Q8_0, 3), (qmm.Q4_K, 6), (qmm.Q6_K, 3)])
def test_fused_quantize_near_rounding_boundaries(qtype, n):
    k = 2048
    x = _near_boundary_rows(np.random.default_rng(124), n)
    x = np.ascontiguousarray(np.tile(x, (1, k // 256)))
    w = synth.gen_weights(qtype, 48, k, np.random.default_rng(125))
    wd, xd = to_dev(w), to_dev(x)
    fused = qmm.matmul(wd, qtype, 48, k, xd)
    xq_dev = qmm.quantize_q8_1(xd)
    assert np.array_equal(xq_dev.cpu().numpy(), oracle.quantize_q8_1(x))
    assert torch.equal(fused, qmm.matmul_q8_1(wd, qtype, 48, k, xq_dev, n))


def test_fused_quantize_special_blocks():
    """Zero blocks, exact rounding ties, a lone spike, a constant block, a subnormal-range scale and
    a scale near the fp16 limit inside the fused kernel's activation rows."""
    blocks = [np.zeros(32), np.concatenate([[15.875, 0.3125, -0.3125, 0.0625, -0.0625, 1.5625], np.zeros(26)]),
              np.where(np.arange(32) == 7, -3.0, 0.0), np.full(32, 0.7), np.linspace(-1e-38, 1e-38, 32),
              np.linspace(-6e4, 6.5e4, 32) * 1e-3, np.concatenate([[127.031005859375, 100.51], np.zeros(30)]),
              np.random.default_rng(570).standard_normal(32)]
    row = np.concatenate(blocks)
    x = np.stack([row, row[::-1].copy(), np.roll(row, 64)]).astype(np.float32)   # k = 256
    for qtype in (qmm.Q4_K, qmm.Q8_0):
        w = synth.gen_weights(qtype, 40, 256, np.random.default_rng(571))
        for n in (1, 2, 3):
            if qtype == qmm.Q4_K and n == 3:
                continue
            xs = np.ascontiguousarray(x[:n])
            wd, xd = to_dev(w), to_dev(xs)
            fused = qmm.matmul(wd, qtype, 40, 256, xd)
            separate = qmm.matmul_q8_1(wd, qtype, 40, 256, qmm.quantize_q8_1(xd), n)
            assert torch.equal(fused, separate), (qtype, n)
            xq = oracle.quantize_q8_1(xs)
            ref = oracle.matmul_q8_1(qtype, w, 40, 256, xq, n)
            assert_close(fused.cpu().numpy(), ref, row_norms(qtype, w, 40, 256), col_norms(xq, n, 256))


def test_matmul_q8_1_entry_matches_matmul():
    qtype, rows, k, n = qmm.Q4_K, 1000, 2048, 24
    w, x = _case(qtype, rows, k, n, 600)
    wd, xd = to_dev(w), to_dev(x)
    y1 = qmm.matmul(wd, qtype, rows, k, xd)
    xq = qmm.quantize_q8_1(xd)
    y2 = qmm.matmul_q8_1(wd, qtype, rows, k, xq, n)
    assert torch.equal(y1, y2)


def test_empty_n_is_noop():
    w, _ = _case(qmm.Q4_K, 64, 256, 1, 610)
    out = torch.full((0, 64), 7.0, device=DEV)
    y = qmm.matmul(to_dev(w), qmm.Q4_K, 64, 256, torch.empty((0, 256), device=DEV), out=out)
    assert y.shape == (0, 64)


def test_wrong_dtype_rejected():
    w, x = _case(qmm.Q4_K, 64, 256, 2, 620)
    with pytest.raises(TypeError):
        qmm.matmul(to_dev(w), qmm.Q4_K, 64, 256, to_dev(x).half())
    with pytest.raises(TypeError):
        qmm.quantize_q8_1(to_dev(x).double())


# ---------------------------------------------------------------------------------------------
# Full-size prefill shapes: sampled outputs
# ---------------------------------------------------------------------------------------------
def _whole_rows_check(y, qtype, w, rows, k, xq, n, rng, nrows=256, what=""):
    """nrows distinct output rows, every column of each, against the oracle run on exactly those
    weight rows (rows always include the first and the last, the edges of the tile grid)."""
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, nrows, replace=False)]))
    rb = oracle.row_bytes(qtype, k)
    wsub = np.ascontiguousarray(w.reshape(rows, rb)[sel])
    ref = oracle.matmul_q8_1(qtype, wsub, len(sel), k, xq, n)
    return assert_close(np.ascontiguousarray(y[:, sel]), ref, row_norms(qtype, wsub, len(sel), k),
                        col_norms(xq, n, k), what=what)


@pytest.mark.parametrize("case", synth.PREFILL_CASES, ids=lambda c: c["name"])
def test_prefill_workloads_whole_rows(case):
    """The prefill projections at full size in the launch configuration the bench times (fp32
    input, automatic plan: stream-K at 512 tokens, whole tiles at 2048)."""
    w, x = synth.make_dense(case)
    qtype, rows, k, n = case["qtype"], case["rows"], case["k"], case["n"]
    y = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    _whole_rows_check(y, qtype, w, rows, k, xq, n, np.random.default_rng(7), what=case["name"])


def test_streamk_on_off_agree_and_rerun_is_bitwise():
    qtype, rows, k, n = qmm.Q6_K, 1024, 14336, 160       # 8 x 2 tiles: stream-K splits every tile
    w, x = _case(qtype, rows, k, n, 700)
    wd, xd = to_dev(w), to_dev(x)
    p = qmm.plan_dense(qtype, rows, k, n)
    assert p["stream_k"] == 1 and p["units"] > p["ntiles"]
    y_sk = qmm.matmul(wd, qtype, rows, k, xd)
    y_sk2 = qmm.matmul(wd, qtype, rows, k, xd)
    assert torch.equal(y_sk, y_sk2)
    qmm.set_override(qmm.OVR_STREAMK, 1)
    y_dp = qmm.matmul(wd, qtype, rows, k, xd)
    xq = oracle.quantize_q8_1(x)
    wn, xn = row_norms(qtype, w, rows, k), col_norms(xq, n, k)
    assert_close(y_sk.cpu().numpy(), y_dp.cpu().numpy(), wn, xn, what="stream-K vs whole tiles")
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    assert_close(y_sk.cpu().numpy(), ref, wn, xn, what="stream-K vs oracle")


@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q6_K, qmm.Q8_0], ids=TNAME.get)
def test_streamk_remainder_after_whole_rounds(qtype):
    """More tiles than units: 40 row tiles x 7 column tiles (the last with 2 live columns) = 280
    tiles on the device's units (256 on this part).  Whole rounds of one tile per unit run
    data-parallel and only the remaining tiles are split by stream-K; every output against the
    oracle, bitwise reruns, and the same products with stream-K off."""
    rows, k, n = 5120, 512, 770
    p = qmm.plan_dense(qtype, rows, k, n)
    assert p["tile_j"] == 128 and p["ntiles"] == 280 and p["stream_k"] == 1
    if p["ntiles"] % p["units"] == 0 or p["units"] >= p["ntiles"]:
        pytest.skip("this device's unit count leaves no remainder after whole rounds")
    w, x = _case(qtype, rows, k, n, 1450 + qtype)
    wd, xd = to_dev(w), to_dev(x)
    y = qmm.matmul(wd, qtype, rows, k, xd)
    assert torch.equal(y, qmm.matmul(wd, qtype, rows, k, xd))
    xq = oracle.quantize_q8_1(x)
    wn, xn = row_norms(qtype, w, rows, k), col_norms(xq, n, k)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    assert_close(y.cpu().numpy(), ref, wn, xn, what=f"{TNAME[qtype]} stream-K remainder")
    qmm.set_override(qmm.OVR_STREAMK, 1)
    y_dp = qmm.matmul(wd, qtype, rows, k, xd)
    assert_close(y.cpu().numpy(), y_dp.cpu().numpy(), wn, xn, what="stream-K remainder vs whole tiles")


@pytest.mark.parametrize("sk", [0, 1], ids=["streamk-auto", "streamk-off"])
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_tile_bands_partial_band_ragged_tiles(qtype, sk):
    """11 row tiles (one full band of 8 and a partial band of 3) x 3 column tiles, the last one
    ragged, with stream-K splitting tiles (auto) or whole tiles (off); every output checked."""
    rows, n = 1300, 300
    k = 544 if qtype == qmm.Q8_0 else 512          # Q8_0: a ragged last 256-value step too
    p = qmm.plan_dense(qtype, rows, k, n)
    assert p["tile_j"] == 128 and p["ntiles"] == 33 and p["stream_k"] == 1
    qmm.set_override(qmm.OVR_STREAMK, sk)
    _full_check(qtype, rows, k, n, 1400 + qtype + sk, f"{TNAME[qtype]} {rows}x{k} n={n} sk={sk}")


@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q8_0], ids=TNAME.get)
def test_few_columns_beyond_matvec_k_limit(qtype):
    """At most 8 columns but K above the matrix-vector kernel's limit: the tiled kernel takes
    the call (with the tiled activation layout)."""
    rows, k, n = 40, 32768 + 256, 3
    assert qmm.plan_dense(qtype, rows, k, n)["regime"] == 2
    _full_check(qtype, rows, k, n, 1500 + qtype, f"{TNAME[qtype]} {rows}x{k} n={n}")


@pytest.mark.parametrize("J", [32, 64, 128])
def test_q4k_min_term_large_dmin(J):
    """Q4_K min coefficients -dmin*m near and beyond the fp16 range: rows 64..127 with dmin = 1000
    (|dmin*m| up to 63000) and rows 128..159 with dmin = 60000 (up to 3.8e6, far beyond fp16).  The
    tiled kernel's min term splits -dmin*m exactly into three bf16 pieces, which keep fp32's
    exponent range, so no coefficient can overflow; every output against the oracle."""
    rows, k, n = 256, 512, 70
    w, x = _case(qmm.Q4_K, rows, k, n, 1600 + J)
    blocks = w.reshape(rows, k // 256, 144)
    blocks[64:128, :, 2:4] = np.frombuffer(np.float16(1000.0).tobytes(), np.uint8)
    blocks[128:160, :, 2:4] = np.frombuffer(np.float16(60000.0).tobytes(), np.uint8)
    qmm.set_override(qmm.OVR_TILE_J, J)
    y = qmm.matmul(to_dev(w), qmm.Q4_K, rows, k, to_dev(x)).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    ref = oracle.matmul_q8_1(qmm.Q4_K, w, rows, k, xq, n)
    assert np.all(np.isfinite(y))
    assert_close(y, ref, row_norms(qmm.Q4_K, w, rows, k), col_norms(xq, n, k), what=f"J={J}")


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_forced_regimes_agree(qtype):
    rows, k, n = 520, 1024, 6
    w, x = _case(qtype, rows, k, n, 800)
    wd, xd = to_dev(w), to_dev(x)
    qmm.set_override(qmm.OVR_PATH, qmm.PATH_MATVEC)
    y_mv = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
    qmm.set_override(qmm.OVR_PATH, qmm.PATH_TILED)
    y_mq = qmm.matmul(wd, qtype, rows, k, xd).cpu().numpy()
    xq = oracle.quantize_q8_1(x)
    wn, xn = row_norms(qtype, w, rows, k), col_norms(xq, n, k)
    ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
    assert_close(y_mv, ref, wn, xn, what="matrix-vector")
    assert_close(y_mq, ref, wn, xn, what="tiled")


@pytest.mark.parametrize("J", [32, 64, 128])
def test_tile_widths(J):
    qtype, rows, k, n = qmm.Q4_K, 384, 1024, 100
    qmm.set_override(qmm.OVR_TILE_J, J)
    _full_check(qtype, rows, k, n, 900 + J, f"J={J}")


# ---------------------------------------------------------------------------------------------
# Expert-indexed product
# ---------------------------------------------------------------------------------------------
def _moe_whole_rows(case, w, x, ids, y, rng, nrows=256):
    """nrows distinct output rows of every (token, slot) pair: the oracle's expert product on the
    same rows of every expert, compared element by element."""
    qtype, rows, k, n_exp = case["qtype"], case["rows"], case["k"], case["n_exp"]
    n_tok, top_k = ids.shape
    xpt = case["x_per_tok"]
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, nrows, replace=False)]))
    rb = oracle.row_bytes(qtype, k)
    wsub = np.ascontiguousarray(w.reshape(n_exp, rows, rb)[:, sel])
    ref, bad = oracle.matmul_id(qtype, wsub, n_exp, len(sel), k, x, xpt, ids)
    assert bad == 0
    xq = oracle.quantize_q8_1(x)
    wn = row_norms(qtype, wsub, n_exp * len(sel), k).reshape(n_exp, len(sel))
    xn = col_norms(xq, xq.shape[0], k)
    got = y[:, :, sel]
    arow = np.arange(n_tok)[:, None] * xpt + (np.arange(top_k)[None, :] if xpt > 1 else 0)
    denom = wn[ids] * xn[arow][:, :, None]
    assert np.all(np.isfinite(got))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64)) / denom
    assert err.max() <= 1e-4, f"max normalised error {err.max():.3e} at {np.unravel_index(np.argmax(err), err.shape)}"
    return float(err.max())


@pytest.mark.parametrize("case", synth.MOE_CASES, ids=lambda c: c["name"])
def test_moe_workloads(case):
    w, x, ids = synth.make_moe(case)
    qtype, n_exp, rows, k = case["qtype"], case["n_exp"], case["rows"], case["k"]
    y, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=case["x_per_tok"])
    assert qmm.matmul_id_invalid_count(ws) == 0
    y = y.cpu().numpy()
    if case["n_tok"] <= 64:
        ref, bad = oracle.matmul_id(qtype, w, n_exp, rows, k, x, case["x_per_tok"], ids)
        assert bad == 0
        xq = oracle.quantize_q8_1(x)
        wn_all = row_norms(qtype, w, n_exp * rows, k).reshape(n_exp, rows)
        xn_all = col_norms(xq, xq.shape[0], k)
        n_tok, top_k = ids.shape
        for t in range(n_tok):
            for s in range(top_k):
                a = t * case["x_per_tok"] + (s if case["x_per_tok"] > 1 else 0)
                assert_close(y[t, s][None], ref[t, s][None], wn_all[ids[t, s]], xn_all[a:a + 1], what=f"pair {t},{s}")
    else:
        _moe_whole_rows(case, w, x, ids, y, np.random.default_rng(11))


def test_moe_invalid_ids_and_per_slot_activations():
    rng = np.random.default_rng(1000)
    n_exp, rows, k, n_tok, top_k = 6, 200, 512, 40, 3
    qtype = qmm.Q4_K
    w = synth.gen_weights(qtype, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok * top_k, k)).astype(np.float32)
    ids = np.stack([rng.choice(n_exp, top_k, replace=False) for _ in range(n_tok)]).astype(np.int32)
    ids[0, 0] = n_exp
    ids[5, 2] = -7
    ids[39, 1] = 1000
    out = torch.full((n_tok, top_k, rows), 12345.0, device=DEV)
    y, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=top_k, out=out)
    assert qmm.matmul_id_invalid_count(ws) == 3
    y = y.cpu().numpy()
    ref, bad = oracle.matmul_id(qtype, w, n_exp, rows, k, x, top_k, ids, fill=12345.0)
    assert bad == 3
    for t, s in [(0, 0), (5, 2), (39, 1)]:
        assert np.all(y[t, s] == 12345.0)
    xq = oracle.quantize_q8_1(x)
    wn_all = row_norms(qtype, w, n_exp * rows, k).reshape(n_exp, rows)
    xn_all = col_norms(xq, n_tok * top_k, k)
    for t in range(n_tok):
        for s in range(top_k):
            e = ids[t, s]
            if 0 <= e < n_exp:
                a = t * top_k + s
                assert_close(y[t, s][None], ref[t, s][None], wn_all[e], xn_all[a:a + 1], what=f"pair {t},{s}")


@pytest.mark.parametrize("deep", [False, True], ids=["k2048", "k_past_16_steps"])
@pytest.mark.parametrize("kernel", [1, 2], ids=MV_KNAME.get)
@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_moe_small_experts_both_kernels(qtype, kernel, deep):
    """Experts with at most 8 columns go to the matrix-vector kernel in expert mode; both kernels,
    ragged rows, per-slot activations, every output against the oracle; K = 2048, and K past 16
    steps (some waves take two)."""
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    rng = np.random.default_rng(1100 + qtype + (7 if deep else 0))
    k = (6144 if qtype == qmm.Q6_K else 4352) if deep else 2048
    n_exp, rows, n_tok, top_k = 6, 77, 20, 2
    w = synth.gen_weights(qtype, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok * top_k, k)).astype(np.float32)
    ids = np.stack([rng.choice(n_exp, top_k, replace=False) for _ in range(n_tok)]).astype(np.int32)
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


@pytest.mark.parametrize("kernel", [1, 2], ids=MV_KNAME.get)
@pytest.mark.parametrize("qtype", [qmm.Q4_K, qmm.Q6_K, qmm.Q8_0], ids=TNAME.get)
def test_moe_small_experts_strided_workgroups(qtype, kernel):
    """Dense routing with a few small experts: more than 16 pairs per expert on average, so the
    matrix-vector launch holds a few grid rows (about four workgroups per compute unit over the
    2048 rows' 128 row groups: 8 rows on 256 compute units) and each row walks the small-expert
    list with that stride, two experts for some workgroups.  Experts 0-3 take 54 pairs each,
    experts 4-15 seven each (small); every output against the oracle, the tiled experts' too.
    K = 256 (one wave per workgroup) except for Q6_K in the LDS-staged kernel, which needs
    16-byte aligned rows (K a multiple of 2048)."""
    qmm.set_override(qmm.OVR_MV_KERNEL, kernel)
    rng = np.random.default_rng(1150 + qtype + kernel)
    n_exp, rows, n_tok, top_k = 16, 2048, 150, 2
    k = 2048 if qtype == qmm.Q6_K and kernel == 2 else 256
    ids = np.zeros((n_tok, top_k), dtype=np.int32)
    for t in range(n_tok):
        ids[t, 0] = t % 4
        ids[t, 1] = 4 + t % 12 if t < 84 else (t + 1) % 4
    counts = np.bincount(ids.reshape(-1), minlength=n_exp)
    assert counts[4:].max() <= 8 and ids.size > 16 * n_exp
    w = synth.gen_weights(qtype, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok, k)).astype(np.float32)
    y, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=1)
    assert qmm.matmul_id_invalid_count(ws) == 0
    y = y.cpu().numpy()
    ref, bad = oracle.matmul_id(qtype, w, n_exp, rows, k, x, 1, ids)
    assert bad == 0
    xq = oracle.quantize_q8_1(x)
    wn_all = row_norms(qtype, w, n_exp * rows, k).reshape(n_exp, rows)
    xn_all = col_norms(xq, n_tok, k)
    for t in range(n_tok):
        for s in range(top_k):
            assert_close(y[t, s][None], ref[t, s][None], wn_all[ids[t, s]], xn_all[t:t + 1], what=f"pair {t},{s}")


def _grouping_ref(ids, n_exp, tile_j, small_max):
    """Host counting sort of the (token, slot) pairs by expert (the expert-bounds passage: each
    expert's pairs contiguous); stable, so each segment is in ascending pair order, against which
    the device's segments are compared as sets."""
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < n_exp)
    p = np.nonzero(valid)[0]
    order = p[np.argsort(flat[p], kind="stable")]
    counts = np.bincount(flat[p], minlength=n_exp)
    bounds = np.concatenate([[0], np.cumsum(counts)])
    tiles, tile_start, small = 0, [], []
    for e in range(n_exp):
        tile_start.append(tiles)
        c = int(counts[e])
        if c > small_max:
            tiles += -(-c // tile_j)
        elif c > 0:
            small.append(e)
    tile_start.append(tiles)
    small += [-1] * (n_exp - len(small))
    return order, bounds, np.array(tile_start), np.array(small), int((~valid).sum())


@pytest.mark.parametrize("n_exp,n_tok,top_k,zipf", [(8, 512, 2, 1.1), (128, 2048, 8, 1.0), (6, 37, 3, 0.0),
                                                     (1000, 333, 4, 0.8), (5000, 50, 2, 0.0),
                                                     (128, 5000, 8, 1.0),    # many batches per wave
                                                     (128, 2049, 8, 1.0),    # just past ids kept in registers
                                                     (1, 100, 1, 0.0),       # one expert: no id bits
                                                     (2304, 700, 4, 0.5),    # the most the wave ranking takes
                                                     (2305, 700, 4, 0.5),    # the per-thread counting beyond
                                                     (64, 3, 5, 0.0)])       # fewer pairs than one wave
def test_moe_grouping_is_a_counting_sort(n_exp, n_tok, top_k, zipf):
    """The device grouping pass (index work: bit-exact) against a host counting sort, including
    invalid ids, ragged chunks and both grouping kernels: segment bounds, tile prefix and the
    small-expert list exactly; each expert's segment holds exactly that expert's pairs (the order
    inside a segment is not unique -- up to 2304 experts the slots come from LDS atomics -- and
    no product depends on it: each column is computed on its own)."""
    rng = np.random.default_rng(1300 + n_exp)
    qtype, rows, k = qmm.Q8_0, 16, 256
    if zipf > 0:
        pr = 1.0 / np.arange(1, n_exp + 1) ** zipf
        pr /= pr.sum()
        ids = np.stack([rng.choice(n_exp, top_k, replace=False, p=pr) for _ in range(n_tok)]).astype(np.int32)
    else:
        ids = rng.integers(0, n_exp, (n_tok, top_k)).astype(np.int32)
    ids.reshape(-1)[rng.integers(0, n_tok * top_k, 5)] = np.array([-1, n_exp, n_exp + 7, -100, 1 << 30], np.int32)
    w = synth.gen_weights(qtype, n_exp * rows, k, rng)
    x = rng.standard_normal((n_tok, k)).astype(np.float32)
    _, ws = qmm.matmul_id(to_dev(w), qtype, n_exp, rows, k, to_dev(x), to_dev(ids), x_per_tok=1)
    g = qmm.matmul_id_grouping(ws, qtype, n_exp, k, n_tok, top_k, 1)
    order, bounds, tile_start, small, bad = _grouping_ref(ids, n_exp, g["tile_j"], g["small_max"])
    assert qmm.matmul_id_invalid_count(ws) == bad
    assert np.array_equal(g["bounds"].numpy(), bounds)
    got = g["sorted"].numpy()[:bounds[-1]]
    for e in range(n_exp):
        seg = slice(bounds[e], bounds[e + 1])
        assert np.array_equal(np.sort(got[seg]), order[seg]), e      # order[] is ascending per expert
    assert np.array_equal(g["tile_start"].numpy(), tile_start)
    assert np.array_equal(g["small"].numpy(), small)


def test_moe_rerun_is_bitwise():
    case = synth.MOE_CASES[3]
    w, x, ids = synth.make_moe(case)
    args = (to_dev(w), case["qtype"], case["n_exp"], case["rows"], case["k"], to_dev(x), to_dev(ids))
    y1, _ = qmm.matmul_id(*args, x_per_tok=case["x_per_tok"])
    y2, _ = qmm.matmul_id(*args, x_per_tok=case["x_per_tok"])
    assert torch.equal(y1, y2)
