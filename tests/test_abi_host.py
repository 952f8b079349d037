"""C-ABI library loading, exported symbols and host-side planner logic (CPU only, no GPU calls).

Planner numbers are the MMQ page's printed arithmetic: "tile efficiency" section (100 tiles on
108 SMs -> 92 %, 120 tiles -> 55 %), "worked example: 8K prefill" (11008 rows x 8192 columns at
I = J = 128 -> 86 x 64 = 5504 tiles; 64 experts, 8192 tokens, top-2 -> 256 tokens per expert),
"J runtime selection" (fewest column tiles, ties to the smaller J) and "stream-K" (unit u owns
[u*W/units, (u+1)*W/units) of the flattened (tile, K-step) items).
"""
import ctypes
import subprocess

import pytest

import block_quantized_matmul_quantize_amd as qmm


def test_library_exports_every_header_symbol():
    declared = qmm.header_symbols()
    assert len(declared) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", qmm.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(qmm.lib(), s)


def test_probe_library_exports_its_header():
    """The benchmark's measurement probes (include/qmm_probe.h) live in their own library."""
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "include", "qmm_probe.h")) as f:
        declared = sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", f.read())))
    assert declared == ["qmm_probe_mfma_i8", "qmm_probe_read"]
    lib = os.path.join(os.path.dirname(qmm.LIB_PATH), "libqmm_probe.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported


def test_version_string():
    assert "gfx950" in qmm.version()


@pytest.mark.parametrize("ntiles,nsm,pct", [(100, 108, 92), (120, 108, 55), (108, 108, 100), (216, 108, 100),
                                            (217, 108, 66), (448, 256, 87), (128, 256, 50), (1, 256, 0)])
def test_tile_efficiency(ntiles, nsm, pct):
    assert qmm.tile_efficiency(ntiles, nsm) == pct


def test_worked_example_tile_count():
    # 11008 rows, 8192 columns, I = J = 128
    assert qmm.select_tile_j(8192) == 128
    rows_tiles = (11008 + 127) // 128
    col_tiles = (8192 + qmm.select_tile_j(8192) - 1) // qmm.select_tile_j(8192)
    assert (rows_tiles, col_tiles, rows_tiles * col_tiles) == (86, 64, 5504)
    p = qmm.plan_dense(qmm.Q4_K, 11008, 4096, 8192, nsm=108)
    assert p["regime"] == 2 and p["tile_j"] == 128 and p["ntiles"] == 5504
    # 5504 tiles is about 51 rounds on 108 units (one 128-column tile resident per unit):
    # efficiency well above the stream-K threshold, so one workgroup per tile
    assert p["stream_k"] == 0 and p["units"] == 5504
    # MoE average: 8192 tokens x top-2 over 64 experts
    assert 8192 * 2 // 64 == 256


@pytest.mark.parametrize("ncols,J", [(1, 32), (16, 32), (32, 32), (33, 64), (64, 64), (65, 128), (100, 128),
                                     (128, 128), (129, 128), (512, 128), (2048, 128)])
def test_select_tile_j(ncols, J):
    assert qmm.select_tile_j(ncols) == J


@pytest.mark.parametrize("qtype,n,J", [
    (qmm.Q4_K, 48, 32), (qmm.Q4_K, 64, 32), (qmm.Q4_0, 40, 32), (qmm.Q5_K, 33, 32),   # two 32-column tiles
    (qmm.Q6_K, 48, 128), (qmm.Q3_K, 64, 128), (qmm.Q8_0, 40, 128),                      # one 128-column tile
    (qmm.Q4_K, 32, 32), (qmm.Q6_K, 20, 32), (qmm.Q4_K, 65, 128), (qmm.Q6_K, 512, 128),  # fewest tiles
])
def test_dense_tile_width_avoids_single_64_column_tile(qtype, n, J):
    """33-64 columns: the 64-column tile measured slowest, so the plan takes one 128-column tile
    for Q6_K / Q3_K / Q8_0 and two 32-column tiles for the other types; elsewhere the fewest."""
    p = qmm.plan_dense(qtype, 4096, 4096, n)
    assert p["regime"] == 2 and p["tile_j"] == J


def test_plan_regimes():
    assert qmm.plan_dense(qmm.Q4_K, 4096, 4096, 1)["regime"] == 1
    assert qmm.plan_dense(qmm.Q4_K, 4096, 4096, 8)["regime"] == 1
    assert qmm.plan_dense(qmm.Q4_K, 4096, 4096, 9)["regime"] == 2
    p = qmm.plan_dense(qmm.Q4_K, 512, 1024, 16)
    assert p["regime"] == 2 and p["tile_j"] == 32 and p["ntiles"] == 4
    # prefill down projection: 32 x 4 tiles underfill 256 units -> stream-K over 256 units
    p = qmm.plan_dense(qmm.Q6_K, 4096, 14336, 512)
    assert p["ntiles"] == 128 and p["stream_k"] == 1 and p["units"] == 256 and p["k_iters"] == 56
    # up projection: 112 x 4 = 448 tiles in two rounds of 256 (87.5 %, below 90 %) -> stream-K
    p = qmm.plan_dense(qmm.Q4_K, 14336, 4096, 512)
    assert p["ntiles"] == 448 and p["efficiency_pct"] == 87 and p["stream_k"] == 1 and p["units"] == 256
    # 2048 tokens: 1792 tiles, exactly seven rounds -> one workgroup per tile
    p = qmm.plan_dense(qmm.Q4_K, 14336, 4096, 2048)
    assert p["ntiles"] == 1792 and p["efficiency_pct"] == 100 and p["stream_k"] == 0 and p["units"] == 1792


def test_overrides_and_restore():
    try:
        qmm.set_override(qmm.OVR_PATH, qmm.PATH_TILED)
        assert qmm.plan_dense(qmm.Q4_K, 4096, 4096, 4)["regime"] == 2
        qmm.set_override(qmm.OVR_STREAMK, 1)
        assert qmm.plan_dense(qmm.Q6_K, 4096, 14336, 512)["stream_k"] == 0
        qmm.set_override(qmm.OVR_TILE_J, 64)
        assert qmm.plan_dense(qmm.Q4_K, 4096, 4096, 512)["tile_j"] == 64
        with pytest.raises(qmm.QmmError):
            qmm.set_override(qmm.OVR_TILE_J, 48)
        with pytest.raises(qmm.QmmError):
            qmm.set_override(99, 1)
    finally:
        for key in (qmm.OVR_PATH, qmm.OVR_STREAMK, qmm.OVR_TILE_J):
            qmm.set_override(key, 0)


@pytest.mark.parametrize("ntiles,k_iters,units", [(128, 56, 256), (448, 16, 256), (5, 7, 3), (1, 16, 16),
                                                  (7, 1, 7), (9, 13, 256)])
def test_streamk_partition_covers_every_item_once(ntiles, k_iters, units):
    units = min(units, ntiles * k_iters)
    W = ntiles * k_iters
    starts = [qmm.streamk_unit_start(u, units, ntiles, k_iters) for u in range(units + 1)]
    assert starts[0] == 0 and starts[-1] == W
    assert all(b > a for a, b in zip(starts, starts[1:]))          # every unit has work
    sizes = [b - a for a, b in zip(starts, starts[1:])]
    assert max(sizes) - min(sizes) <= 1                              # balanced
    covered = [0] * W
    for a, b in zip(starts, starts[1:]):
        for i in range(a, b):
            covered[i] += 1
    assert covered == [1] * W
    # a unit touches at most two partial tiles (its first and its last)
    for a, b in zip(starts, starts[1:]):
        tiles = range(a // k_iters, (b - 1) // k_iters + 1)
        partial = [t for t in tiles if max(a, t * k_iters) > t * k_iters or min(b, (t + 1) * k_iters) < (t + 1) * k_iters]
        assert len(partial) <= 2
        assert all(t in (tiles[0], tiles[-1]) for t in partial)


def _status(fn, *args):
    return fn(*args)


def test_argument_validation_without_gpu():
    L = qmm.lib()
    null = ctypes.c_void_p(0)
    # unsupported type
    assert L.qmm_matmul(3, null, 16, 256, null, 1, null, null, 0, null) == -2
    assert b"unsupported" in L.qmm_last_error()
    # k not a multiple of the block size
    assert L.qmm_matmul(qmm.Q4_K, null, 16, 100, null, 1, null, null, 0, null) == -3
    assert L.qmm_matmul(qmm.Q8_0, null, 16, 48, null, 1, null, null, 0, null) == -3
    assert L.qmm_quantize_q8_1(null, 1, 33, null, null) == -3
    # negative sizes, null pointers
    assert L.qmm_matmul(qmm.Q4_K, null, 0, 256, null, 1, null, null, 0, null) == -1
    assert L.qmm_matmul(qmm.Q4_K, null, 16, 256, null, -1, null, null, 0, null) == -1
    assert L.qmm_matmul(qmm.Q4_K, null, 16, 256, null, 1, null, null, 0, null) == -1
    # n == 0 is a no-op
    assert L.qmm_matmul(qmm.Q4_K, null, 16, 256, null, 0, null, null, 0, null) == 0
    assert L.qmm_quantize_q8_1(null, 0, 32, null, null) == 0
    # bad x_per_tok / top_k
    assert L.qmm_matmul_id(qmm.Q4_K, null, 4, 16, 256, null, 3, null, 8, 2, null, null, 0, null) == -1
    assert L.qmm_matmul_id(qmm.Q4_K, null, 4, 16, 256, null, 1, null, 8, 0, null, null, 0, null) == -1
    # debug export: bad path, too many columns for the matrix-vector kernel, workspace too small
    one = ctypes.c_void_p(4096)   # a non-null address, never dereferenced: the calls fail first
    assert L.qmm_debug_subdots(qmm.Q4_K, null, 16, 256, null, 1, 3, null, null, 0, null) == -1
    assert L.qmm_debug_subdots(qmm.Q4_K, null, 16, 256, null, 9, 1, null, null, 0, null) == -1
    assert qmm.debug_subdots_workspace(qmm.Q4_K, 16, 256, 9, qmm.PATH_TILED) > 0
    assert L.qmm_debug_subdots(qmm.Q4_K, one, 16, 256, one, 9, 2, one, null, 0, null) == -4


def test_glu_argument_validation_without_gpu():
    L = qmm.lib()
    null = ctypes.c_void_p(0)
    one = ctypes.c_void_p(4096)   # a non-null address, never dereferenced: the calls fail first
    assert L.qmm_matmul_glu(3, null, null, 16, 256, null, 1, null, null, 0, null) == -2
    assert L.qmm_matmul_glu(qmm.Q4_K, null, null, 16, 100, null, 1, null, null, 0, null) == -3
    assert L.qmm_matmul_glu(qmm.Q4_K, null, null, 16, 256, null, 0, null, null, 0, null) == 0
    # null up matrix with columns to compute
    assert L.qmm_matmul_glu(qmm.Q4_K, one, null, 16, 256, one, 1, one, null, 0, null) == -1
    assert b"w_up" in L.qmm_last_error()
    # workspace too small (host check, before any launch)
    assert L.qmm_matmul_glu(qmm.Q4_K, one, one, 16, 256, one, 1, one, null, 0, null) == -4
    assert L.qmm_matmul_id_glu(qmm.Q4_K, one, null, 4, 16, 256, one, one, 8, 2, one, null, 0, null) == -1
    assert L.qmm_matmul_id_glu(qmm.Q4_K, null, null, 4, 16, 256, null, null, 8, 0, null, null, 0, null) == -1


def test_glu_workspace_sizes():
    # matrix-vector form: the q8_1 copy of x; tiled form: the tiled activation layout, no partials
    assert qmm.matmul_glu_workspace(qmm.Q4_K, 4096, 4096, 3) >= 3 * 4096 // 32 * 36
    assert qmm.matmul_glu_workspace(qmm.Q4_K, 14336, 4096, 512) >= 512 * 4096 // 32 * 36
    assert qmm.matmul_glu_workspace(qmm.Q4_K, 14336, 4096, 512) < qmm.matmul_workspace(qmm.Q4_K, 14336, 4096, 512)
    assert qmm.matmul_id_glu_workspace(qmm.Q4_K, 8, 768, 2048, 64, 8) == \
        qmm.matmul_id_workspace(qmm.Q4_K, 8, 768, 2048, 64, 8, 1)


def test_workspace_sizes_monotone():
    # matrix-vector from q8_1 input needs no workspace; from fp32 it holds the q8_1 codes
    assert qmm.matmul_q8_1_workspace(qmm.Q4_K, 4096, 4096, 1) == 0
    assert qmm.matmul_workspace(qmm.Q4_K, 4096, 4096, 1) >= 4096 // 32 * 36
    # the tiled path reserves stream-K partial slots
    assert qmm.matmul_q8_1_workspace(qmm.Q6_K, 4096, 14336, 512) >= 256 * 2 * 128 * 128 * 4
    assert qmm.matmul_workspace(3, 16, 256, 1) == 0
    assert qmm.matmul_id_workspace(qmm.Q4_K, 8, 14336, 4096, 512, 2, 1) > 512 * 128 * 36
    assert qmm.matmul_id_workspace(qmm.Q4_K, 8, 14336, 4096, 512, 2, 3) == 0


MV_AUTO = [
    # (type, rows, n, expected (kernel, fused)) for aligned weights and fp32 activations, K = 4096:
    # dot4 for Q4_K, Q5_K and Q4_0 at n <= 3 from 8192 rows on (Q8_0: n = 1 from 8192 rows, n <= 3
    # from 12288), else the LDS-staged kernel; both quantize the fp32 input themselves at every
    # n <= 8.
    *[(t, 4096, n, (2, True)) for t in (qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0) for n in range(1, 9)],
    *[(t, 8192, 1, (3, True)) for t in (qmm.Q4_K, qmm.Q5_K, qmm.Q8_0, qmm.Q4_0)],
    *[(t, 8192, n, (3, True)) for t in (qmm.Q4_K, qmm.Q5_K, qmm.Q4_0) for n in (2, 3)],
    *[(t, 8192, 4, (2, True)) for t in (qmm.Q4_K, qmm.Q5_K, qmm.Q8_0, qmm.Q4_0)],
    *[(qmm.Q8_0, r, n, (2, True)) for r in (8192, 12287) for n in (2, 3)],
    *[(qmm.Q8_0, r, n, (3, True)) for r in (12288, 14336) for n in (2, 3)],
    (qmm.Q4_K, 8191, 1, (2, True)),
    (qmm.Q6_K, 14336, 1, (2, True)),
    *[(t, 14336, 2, (3, True)) for t in (qmm.Q4_K, qmm.Q8_0)],
    *[(t, 4096, 9, (0, False)) for t in (qmm.Q4_K, qmm.Q5_K, qmm.Q6_K, qmm.Q8_0, qmm.Q4_0)],
    # Q3_K and IQ4_XS: dot4 up to three columns at any row count, then quantize + register-streamed
    *[(t, r, n, (3, True)) for t in (qmm.Q3_K, qmm.IQ4_XS) for r in (16, 4096, 14336) for n in (1, 2, 3)],
    *[(t, 4096, n, (1, False)) for t in (qmm.Q3_K, qmm.IQ4_XS) for n in (4, 8)],
]


@pytest.mark.parametrize("qtype,rows,n,expect", MV_AUTO)
def test_matvec_kernel_automatic_choice(qtype, rows, n, expect):
    assert qmm.matvec_kernel(qtype, 0x10000, rows, 4096, 0x20000, n, x_fp32=True) == expect


def test_matvec_kernel_choice_follows_alignment_and_overrides():
    mk = lambda t, w, k, x, n, rows=8192, **kw: qmm.matvec_kernel(t, w, rows, k, x, n, **kw)
    # q8_1 input: 4-byte alignment serves both dot4 and the LDS-staged kernel, 2-byte neither
    assert mk(qmm.Q4_K, 0x10000, 4096, 0x20004, 1, x_fp32=False) == (3, False)
    assert mk(qmm.Q4_K, 0x10000, 4096, 0x20004, 1, rows=4096, x_fp32=False) == (2, False)
    assert mk(qmm.Q4_K, 0x10000, 4096, 0x20004, 5, x_fp32=False) == (2, False)
    assert mk(qmm.Q4_K, 0x10000, 4096, 0x20002, 1, x_fp32=False) == (1, False)
    assert mk(qmm.Q6_K, 0x10000, 4096, 0x20002, 5, x_fp32=False) == (1, False)
    # weights only 2-byte aligned: the register-streamed kernel, on the quantized copy
    assert mk(qmm.Q4_K, 0x10002, 4096, 0x20000, 1, x_fp32=True) == (1, False)
    assert mk(qmm.Q6_K, 0x10002, 4096, 0x20000, 4, x_fp32=True) == (1, False)
    # Q8_0 weights need 4-byte alignment in both kernels (Q4_K / Q6_K: 16 in the LDS-staged one)
    assert mk(qmm.Q8_0, 0x10004, 4096, 0x20000, 1, x_fp32=True) == (3, True)
    assert mk(qmm.Q8_0, 0x10004, 4096, 0x20000, 5, x_fp32=True) == (2, True)
    assert mk(qmm.Q8_0, 0x10002, 4096, 0x20000, 6, x_fp32=True) == (1, False)
    assert mk(qmm.Q6_K, 0x10004, 4096, 0x20000, 6, x_fp32=True) == (1, False)
    # Q3_K / IQ4_XS: dot4 reads any 2-byte aligned rows
    assert mk(qmm.Q3_K, 0x10002, 4096, 0x20000, 2, x_fp32=True) == (3, True)
    assert mk(qmm.IQ4_XS, 0x10002, 4096, 0x20002, 3, x_fp32=False) == (1, False)
    assert mk(qmm.IQ4_XS, 0x10002, 4096, 0x20004, 3, x_fp32=False) == (3, False)
    # K not a multiple of 256 (Q8_0 allows multiples of 32): register-streamed
    assert mk(qmm.Q8_0, 0x10000, 4128, 0x20000, 2, x_fp32=True) == (1, False)
    with pytest.raises(qmm.QmmError):
        mk(qmm.Q4_K, 0x10000, 4096, 0x20004, 1, x_fp32=True)   # fp32 x must be 16-byte aligned
    try:
        qmm.set_override(qmm.OVR_MV_KERNEL, 1)
        assert mk(qmm.Q4_K, 0x10000, 4096, 0x20000, 1) == (1, False)
        qmm.set_override(qmm.OVR_MV_KERNEL, 2)
        assert mk(qmm.Q4_K, 0x10000, 4096, 0x20000, 1) == (2, True)
        qmm.set_override(qmm.OVR_MV_KERNEL, 3)
        assert mk(qmm.Q4_K, 0x10000, 4096, 0x20000, 1, rows=16) == (3, True)
        qmm.set_override(qmm.OVR_MV_KERNEL, 0)
        qmm.set_override(qmm.OVR_FUSE_COLS, 2)
        assert mk(qmm.Q6_K, 0x10000, 4096, 0x20000, 3) == (2, False)
        qmm.set_override(qmm.OVR_FUSE_COLS, 0)
        qmm.set_override(qmm.OVR_PATH, 2)
        assert mk(qmm.Q4_K, 0x10000, 4096, 0x20000, 1) == (0, False)
    finally:
        for key in (qmm.OVR_MV_KERNEL, qmm.OVR_FUSE_COLS, qmm.OVR_PATH):
            qmm.set_override(key, 0)


@pytest.mark.parametrize("qtype,n_exp,n_tok,top_k,J", [
    (qmm.Q6_K, 128, 2048, 8, 128),     # Q6_K keeps 128-column tiles
    (qmm.Q4_K, 128, 2048, 8, 32),      # mean 128, typical = mean/4 = 32
    (qmm.Q4_K, 8, 512, 2, 32),         # mean 128, typical 32
    (qmm.Q4_K, 16, 384, 2, 32),        # mean 48
    (qmm.Q4_K, 8, 800, 2, 64),         # mean 200, typical 50
    (qmm.Q4_K, 8, 1040, 2, 128),       # mean 260, typical 65
    (qmm.Q8_0, 64, 100, 4, 32),        # mean 6
    (qmm.Q4_K, 4, 1024, 2, 128),       # mean 512
])
def test_expert_tile_width_follows_typical_columns_per_expert(qtype, n_exp, n_tok, top_k, J):
    lay = qmm.matmul_id_layout(qtype, n_exp, 2048, n_tok, top_k, 1)
    assert lay[4] == J
    assert lay[5] == 8                                     # experts of <= 8 columns: matrix-vector
    assert qmm.matmul_id_layout(qtype, n_exp, 256 * 1024, n_tok, top_k, 1)[5] == 0   # beyond its K limit
    offs = lay[:4]
    assert all(o % 256 == 0 for o in offs) and list(offs) == sorted(offs)
    assert offs[-1] < qmm.matmul_id_workspace(qtype, n_exp, 64, 2048, n_tok, top_k, 1)
    qmm.set_override(qmm.OVR_TILE_J, 32)
    try:
        assert qmm.matmul_id_layout(qtype, n_exp, 2048, n_tok, top_k, 1)[4] == 32
    finally:
        qmm.set_override(qmm.OVR_TILE_J, 0)


def test_wrappers_refuse_undersized_tensors_without_gpu():
    """The C ABI receives bare pointers, so the binding checks that every weight, activation and
    output tensor holds the bytes its shape needs before any pointer reaches the library (CPU
    tensors here: the size checks come before the device check, nothing is launched)."""
    import torch
    rows, k = 32, 512
    wb = qmm.weight_bytes(qmm.Q4_K, rows, k)
    assert wb == rows * 2 * 144
    w_ok, w_small = torch.zeros(wb, dtype=torch.uint8), torch.zeros(wb - 1, dtype=torch.uint8)
    x = torch.zeros((3, k), dtype=torch.float32)
    with pytest.raises(ValueError, match="w holds"):
        qmm.matmul(w_small, qmm.Q4_K, rows, k, x)
    with pytest.raises(ValueError, match="out holds"):
        qmm.matmul(w_ok, qmm.Q4_K, rows, k, x, out=torch.zeros((3, rows - 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="w holds"):
        qmm.matmul_f16act(w_small, qmm.Q4_K, rows, k, x)
    with pytest.raises(ValueError, match="w holds"):
        qmm.matmul_q8_1(w_small, qmm.Q4_K, rows, k, torch.zeros(3 * 16 * 36, dtype=torch.uint8), 3)
    with pytest.raises(ValueError, match="w_gate holds"):
        qmm.matmul_glu(w_small, w_small, qmm.Q4_K, rows, k, x)
    ids = torch.zeros((3, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="w holds"):
        qmm.matmul_id(torch.zeros(4 * wb - 1, dtype=torch.uint8), qmm.Q4_K, 4, rows, k, x, ids)
    with pytest.raises(ValueError, match="out holds"):
        qmm.matmul_id(torch.zeros(4 * wb, dtype=torch.uint8), qmm.Q4_K, 4, rows, k, x, ids,
                      out=torch.zeros((3, 2, rows - 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="w_gate holds"):
        qmm.matmul_id_glu(w_ok, w_ok, qmm.Q4_K, 4, rows, k, x, ids)
    with pytest.raises(ValueError, match="out holds"):
        qmm.quantize_q8_1(x, out=torch.zeros(3 * 16 * 36 - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="not a positive multiple"):
        qmm.weight_bytes(qmm.Q6_K, rows, 300)
    # correctly sized CPU tensors pass every size check and stop at the device check
    with pytest.raises(ValueError, match="device tensor"):
        qmm.matmul(w_ok, qmm.Q4_K, rows, k, x)


def test_plan_and_workspace_come_from_one_reading_of_the_overrides():
    """Writers flip the path and tile-width overrides while readers plan calls: every plan is one
    of the two consistent (regime, tile width, workspace) combinations, never a mixture -- the
    workspace layout and the regime of a call are derived from the same snapshot."""
    import threading
    rows, k, n = 4096, 4096, 4
    mv_ws = qmm.matmul_workspace(qmm.Q4_K, rows, k, n)
    legal = set()
    try:
        for path in (0, 2):
            for tj in (0, 32, 64, 128):
                qmm.set_override(qmm.OVR_PATH, path)
                qmm.set_override(qmm.OVR_TILE_J, tj)
                p = qmm.plan_dense(qmm.Q4_K, rows, k, n)
                legal.add((p["regime"], p["tile_j"], p["ntiles"], p["ws_bytes"]))
        qmm.set_override(qmm.OVR_PATH, 0)
        qmm.set_override(qmm.OVR_TILE_J, 0)
        assert (1, 8, 256, mv_ws) in legal and len(legal) == 4   # tile width 0 and 32 coincide
        stop = threading.Event()
        seen, errors = [], []

        def writer(i):
            j = 0
            while not stop.is_set():
                qmm.set_override(qmm.OVR_PATH, (0, 2)[(i + j) % 2])
                qmm.set_override(qmm.OVR_TILE_J, (0, 32, 64, 128)[(i * 3 + j) % 4])
                j += 1

        def reader():
            try:
                for _ in range(3000):
                    p = qmm.plan_dense(qmm.Q4_K, rows, k, n)
                    seen.append((p["regime"], p["tile_j"], p["ntiles"], p["ws_bytes"]))
            except Exception as e:   # noqa: BLE001 -- reported below
                errors.append(e)

        ws = [threading.Thread(target=writer, args=(i,)) for i in range(2)]
        rs = [threading.Thread(target=reader) for _ in range(4)]
        for t in ws + rs:
            t.start()
        for t in rs:
            t.join()
        stop.set()
        for t in ws:
            t.join()
        assert not errors, errors
        assert set(seen) <= legal
        assert len(seen) == 4 * 3000
    finally:
        qmm.set_override(qmm.OVR_PATH, 0)
        qmm.set_override(qmm.OVR_TILE_J, 0)


def test_noalloc_entry_refuses_calls_beyond_its_scratch_without_gpu():
    """The allocation-free entry point checks its plan's workspace against its fixed scratch size on
    the host, before any device call (fake addresses here: nothing is launched or looked up)."""
    L = qmm.lib()
    w, x, y = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    assert L.qmm_matmul_noalloc(qmm.Q6_K, w, 4096, 14336, x, 65536, y, None) == -4
    assert b"allocation-free" in L.qmm_last_error()
    assert L.qmm_matmul_noalloc(3, w, 4096, 256, x, 4, y, None) == -2
    assert L.qmm_matmul_noalloc(qmm.Q4_K, w, 4096, 4096, ctypes.c_void_p(0x200004), 4, y, None) == -1
    assert L.qmm_matmul_noalloc(qmm.Q4_K, w, 4096, 4096, x, 0, y, None) == 0


def test_panel_entry_points_check_arguments_without_gpu():
    """The panel-layout calls refuse bad shapes, types and pointers on the host, before any launch;
    their sizes follow the layout (the original bytes of whole 16-row groups)."""
    L = qmm.lib()
    assert qmm.repack_bytes(qmm.Q4_K, 4096, 4096) == 4096 * 4096 // 256 * 144
    assert qmm.repack_bytes(qmm.Q6_K, 17, 512) == 2 * 2 * 16 * 210          # 2 row groups x 2 steps
    assert qmm.repack_bytes(qmm.Q8_0, 16, 96) == 0                           # k % 256 != 0
    assert qmm.repack_bytes(3, 16, 256) == 0                                 # unsupported type
    assert qmm.repack_bytes(qmm.Q4_K, 0, 256) == 0
    assert L.qmm_repack(qmm.Q4_K, None, 16, 256, None, 0, None) == -1       # null pointers
    assert L.qmm_repack(qmm.Q8_0, 2, 16, 96, 16, 1 << 20, None) == -3       # k % 256 != 0
    assert L.qmm_repack(7, 2, 16, 256, 16, 1 << 20, None) == -2             # type
    assert L.qmm_repack(qmm.Q4_K, 2, 16, 256, 24, 1 << 20, None) == -1      # wp not 16-byte aligned
    assert L.qmm_repack(qmm.Q4_K, 2, 16, 256, 32, 100, None) == -1          # wp too small
    assert L.qmm_matmul_packed(qmm.Q4_K, 32, 16, 320, 16, 1, 16, None, 0, None) == -3
    assert L.qmm_matmul_packed(qmm.Q4_K, 24, 16, 256, 16, 1, 16, None, 0, None) == -1   # wp alignment
    assert L.qmm_matmul_packed(qmm.Q4_K, 32, 16, 256, 16, 0, 16, None, 0, None) == 0    # n = 0: no-op
    # the tiled path needs the same workspace as qmm_matmul_q8_1 (tiled activations + partials);
    # up to 8 columns none
    assert qmm.matmul_packed_workspace(qmm.Q4_K, 4096, 4096, 8) == 0
    assert qmm.matmul_packed_workspace(qmm.Q4_K, 4096, 4096, 512) == \
        L.qmm_matmul_q8_1_workspace(qmm.Q4_K, 4096, 4096, 512)
    assert L.qmm_matmul_packed(qmm.Q4_K, 32, 4096, 4096, 16, 512, 16, 256, 256, None) == -4   # workspace
