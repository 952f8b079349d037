"""Helpers shared by the GPU parity tests: device transfer and the normalised tolerance.

Tolerance: |Y_gpu - Y_oracle| <= 1e-4 * ||w_r|| * ||x_n|| for every (column n, row r), with w_r the
fp64 dequantized weight row and x_n the fp64 dequantized q8_1 activation row (d * q).  By
Cauchy-Schwarz ||w_r||*||x_n|| bounds |Y|, so this is a relative bound on the fp32 scale fixups
and accumulation, which are the only inexact steps (the MMQ page, "write-back" section).
"""
import numpy as np
import torch

import oracle

TOL = 1e-4
DEV = "cuda:0"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def row_norms(qtype, w, rows, k, chunk=1024):
    rb = oracle.row_bytes(qtype, k)
    w2 = np.ascontiguousarray(w).reshape(rows, rb)
    out = np.empty(rows, dtype=np.float64)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = np.linalg.norm(oracle.dequantize(qtype, w2[r0:r1], r1 - r0, k), axis=1)
    return out


def col_norms(xq, n, k):
    X, _, _ = oracle.dequantize_q8_1(xq, n, k)
    return np.linalg.norm(X, axis=1)


def normalised_error(y_gpu, y_ref, wn, xn):
    """Elementwise |diff| / (||w_r|| * ||x_n||) for y [n, rows] (wn: [rows], xn: [n])."""
    denom = np.outer(xn, wn)
    denom = np.where(denom > 0, denom, 1.0)
    return np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64)) / denom


def assert_close(y_gpu, y_ref, wn, xn, tol=TOL, what=""):
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    err = normalised_error(y_gpu, y_ref, wn, xn)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"{what}: max normalised error {err.max():.3e} at {worst}"
    return float(err.max())
