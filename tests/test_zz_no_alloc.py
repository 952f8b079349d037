"""The allocation-free dense entry point (qmm_matmul_noalloc, workspace in the library's own
per-GPU scratch buffer) against qmm_matmul with a caller workspace, through the C ABI: the same
plan and kernels, so the outputs must be identical bit for bit, and both within the normalised
1e-4 bound of the oracle.  Calls in a row share the scratch buffer: a large call (stream-K
partials and the tiled activations fill ~42 MB of it), then smaller ones that reuse it with a
different layout, then the large one again."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_quantize_amd as qmm
import oracle
import synth
from gpu_util import assert_close, col_norms, row_norms, to_dev

pytestmark = pytest.mark.gpu


def _inputs(qtype, rows, k, n, seed):
    g_w, g_x = synth.rngs(seed, 2)
    return synth.gen_weights(qtype, rows, k, g_w), synth.gen_activations(n, k, g_x)


def _against_matmul_and_oracle(qtype, rows, k, n, seed, whole=True):
    w, x = _inputs(qtype, rows, k, n, seed)
    wd, xd = to_dev(w), to_dev(x)
    y_na = qmm.matmul_noalloc(wd, qtype, rows, k, xd)
    y_ws = qmm.matmul(wd, qtype, rows, k, xd)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws), f"{qtype} {rows}x{k} n={n}: differs from qmm_matmul"
    xq = oracle.quantize_q8_1(x)
    if whole:
        ref = oracle.matmul_q8_1(qtype, w, rows, k, xq, n)
        assert_close(y_na.cpu().numpy(), ref, row_norms(qtype, w, rows, k), col_norms(xq, n, k))
    else:   # 256 whole rows (every column) of a full-size call
        sel = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(seed).choice(rows, 256, replace=False)]))
        wsub = np.ascontiguousarray(w.reshape(rows, -1)[sel])
        ref = oracle.matmul_q8_1(qtype, wsub, len(sel), k, xq, n)
        assert_close(np.ascontiguousarray(y_na.cpu().numpy()[:, sel]), ref, row_norms(qtype, wsub, len(sel), k),
                     col_norms(xq, n, k))
    return y_na


def test_noalloc_two_calls_second_smaller():
    big = (qmm.Q6_K, 4096, 14336, 512)        # stream-K plan: partial slots + tiled activations
    p = qmm.plan_dense(*big)
    assert p["regime"] == 2 and p["stream_k"] == 1
    y1 = _against_matmul_and_oracle(*big, seed=2001, whole=False)
    _against_matmul_and_oracle(qmm.Q4_K, 1000, 2048, 24, seed=2002)   # smaller tiled call
    _against_matmul_and_oracle(qmm.Q8_0, 300, 1024, 3, seed=2003)     # matrix-vector call
    y1b = _against_matmul_and_oracle(*big, seed=2001, whole=False)    # the large call again
    assert torch.equal(y1, y1b)


def test_noalloc_under_overrides_and_n0():
    qmm.set_override(qmm.OVR_MV_KERNEL, 1)            # register-streamed: q8_1 copy in the scratch
    try:
        _against_matmul_and_oracle(qmm.Q4_K, 77, 4352, 5, seed=2004)
    finally:
        qmm.set_override(qmm.OVR_MV_KERNEL, 0)
    qmm.set_override(qmm.OVR_STREAMK, 2)              # stream-K forced on a small call
    try:
        _against_matmul_and_oracle(qmm.Q5_K, 300, 2048, 70, seed=2005)
    finally:
        qmm.set_override(qmm.OVR_STREAMK, 0)
    w, _ = _inputs(qmm.Q4_K, 64, 256, 1, 2006)
    out = torch.full((0, 64), 7.0, device="cuda:0")
    qmm.matmul_noalloc(to_dev(w), qmm.Q4_K, 64, 256, torch.empty((0, 256), device="cuda:0"), out=out)
