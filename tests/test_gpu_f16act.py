"""GPU parity of the fp16-activation matrix-vector mode (GP100 MMVQ page, "How" step 1) against
the oracle, through the C ABI: encoder bit-exact (fp16 patterns and prescale exponents), block
sums within fp32 rounding, products within the normalised 1e-4 bound at small and full sizes,
edge cases and refusals."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import DEV, assert_close, row_norms, to_dev

pytestmark = pytest.mark.gpu

TYPES = [qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0]
TNAME = {qmm.Q4_K: "q4_K", qmm.Q5_K: "q5_K", qmm.Q6_K: "q6_K", qmm.Q8_0: "q8_0", qmm.Q4_0: "q4_0"}


def _wide_x(n, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, k)) * 2.0 ** rng.integers(-40, 40, (n, k // 32)).repeat(32, axis=1)
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = np.float32(1e-45)
    x[0, 64] = np.float32(1e30)
    x[0, 96:128] = 2.0 ** 14
    x[0, 128:160] = -(2.0 ** 15)
    return x


@pytest.mark.parametrize("n,k,seed", [(3, 512, 1), (8, 4096, 2), (5, 14336, 3)])
def test_encoder_bit_exact(n, k, seed):
    x = _wide_x(n, k, seed) if seed == 1 else np.random.default_rng(seed).standard_normal((n, k)).astype(np.float32)
    y16, e, s = qmm.encode_f16act(to_dev(x))
    torch.cuda.synchronize()
    ry, re, rs = oracle.f16act_encode(x)
    assert np.array_equal(y16.cpu().numpy().view(np.uint16), ry)
    assert np.array_equal(e.cpu().numpy(), re)
    absum = np.abs(ry.view(np.float16).astype(np.float64)).reshape(n, k // 32, 32).sum(axis=2)
    assert np.all(np.abs(s.cpu().numpy().astype(np.float64) - rs) <= 2.0 ** -19 * absum)


def _binade_x(n, k, seed):
    """Column c: every 32-value block at its own power-of-two scale 2^(s_c + 5*(b mod 3)), s_c from
    -60 to +60 over the columns.  Inside a column the blocks span 2^10, so each block's share of a
    dot is at least ~2^-10 of the largest: a block unscaled by a neighbour's exponent (off by 2^5 or
    2^10) moves the result by far more than the per-block bound below allows."""
    rng = np.random.default_rng(seed)
    nb = k // 32
    s_c = np.linspace(-60, 60, n).round().astype(int)
    e = s_c[:, None] + 5 * (np.arange(nb)[None, :] % 3)
    return (rng.standard_normal((n, k)) * np.exp2(e).repeat(32, axis=1)).astype(np.float32)


def _check(qtype, rows, k, n, seed, x=None, per_block=False):
    """Products within 1e-4 of the oracle, normalised by ||w_r|| * ||x_n|| or (per_block) by the
    tighter sum over 32-value blocks b of ||w_r,b|| * ||x_n,b||, which scores every block against
    its own magnitude rather than the column's largest."""
    g_w, g_x = synth.rngs(seed, 2)
    w = synth.gen_weights(qtype, rows, k, g_w)
    if x is None:
        x = synth.gen_activations(n, k, g_x)
    n = x.shape[0]
    y = qmm.matmul_f16act(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy()
    ref = oracle.matmul_f16act(qtype, w, rows, k, x)
    what = f"{TNAME[qtype]} {rows}x{k} n={n}"
    if not per_block:
        assert_close(y, ref, row_norms(qtype, w, rows, k), np.linalg.norm(x.astype(np.float64), axis=1), what=what)
        return
    W = oracle.dequantize(qtype, w, rows, k).reshape(rows, k // 32, 32)
    X = x.astype(np.float64).reshape(n, k // 32, 32)
    denom = np.einsum("rb,nb->nr", np.linalg.norm(W, axis=2), np.linalg.norm(X, axis=2))
    assert np.all(np.isfinite(y)), what
    err = np.abs(y.astype(np.float64) - ref) / np.where(denom > 0, denom, 1.0)
    assert err.max() <= 1e-4, f"{what}: max per-block normalised error {err.max():.3e}"


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 3, 8])
def test_f16act_small_ragged(qtype, n):
    # 77 rows: the last workgroup holds one live wave of four; K = 2304 / 2336: 72 / 73 blocks,
    # so lanes 8+ (or 9+) take one block and the rest two
    k = 2336 if qtype in (qmm.Q8_0, qmm.Q4_0) else 2304
    _check(qtype, 77, k, n, 700 + 10 * qtype + n)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_f16act_wide_range_activations(qtype):
    _check(qtype, 40, 512, 3, 800 + qtype, x=_wide_x(3, 512, 800 + qtype), per_block=True)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
def test_f16act_per_block_exponents_across_binades(qtype):
    _check(qtype, 40, 2048, 8, 850 + qtype, x=_binade_x(8, 2048, 850 + qtype), per_block=True)


@pytest.mark.parametrize("qtype", TYPES, ids=TNAME.get)
@pytest.mark.parametrize("n", [1, 8])
def test_f16act_full_size(qtype, n):
    _check(qtype, 4096, 4096, n, 900 + 10 * qtype + n)


def test_f16act_zero_activations_and_n0():
    w = synth.gen_weights(qmm.Q4_K, 16, 256, synth.rngs(5, 1)[0])
    y = qmm.matmul_f16act(to_dev(w), qmm.Q4_K, 16, 256, torch.zeros((2, 256), dtype=torch.float32, device=DEV))
    assert torch.count_nonzero(y).item() == 0
    out = torch.full((0, 16), 7.0, device=DEV)
    qmm.matmul_f16act(to_dev(w), qmm.Q4_K, 16, 256, torch.zeros((0, 256), dtype=torch.float32, device=DEV), out=out)


def test_f16act_more_accurate_than_q8_1_on_device():
    qtype, rows, k, n = qmm.Q4_K, 256, 4096, 4
    g_w, g_x = synth.rngs(950, 2)
    w = synth.gen_weights(qtype, rows, k, g_w)
    x = synth.gen_activations(n, k, g_x)
    exact = x.astype(np.float64) @ oracle.dequantize(qtype, w, rows, k).T
    y16 = qmm.matmul_f16act(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy().astype(np.float64)
    y8 = qmm.matmul(to_dev(w), qtype, rows, k, to_dev(x)).cpu().numpy().astype(np.float64)
    def rel(y):
        return np.sqrt(((y - exact) ** 2).sum() / (exact ** 2).sum())
    assert rel(y16) < 2e-3 and rel(y8) > 5 * rel(y16)


@pytest.mark.parametrize("qtype,rows,k,n,off", [(qmm.Q4_K, 16, 256, 9, 0),      # more than 8 columns
                                                (3, 16, 256, 1, 0),            # unsupported type
                                                (qmm.Q4_K, 16, 288, 1, 0),     # K not a multiple of 256
                                                (qmm.Q4_K, 16, 256, 1, 2)])    # weights not 16-byte aligned
def test_f16act_refusals(qtype, rows, k, n, off):
    wt = qtype if qtype != 3 else qmm.Q4_K
    kk = k if k % 256 == 0 else 512
    w = to_dev(np.zeros(off + oracle.row_bytes(wt, kk) * rows + 64, np.uint8))[off:]
    with pytest.raises(qmm.QmmError):
        qmm.matmul_f16act(w, qtype, rows, k, torch.zeros((n, k), dtype=torch.float32, device=DEV))
