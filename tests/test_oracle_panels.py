"""Pins for the oracle's panel repack (CPU only).

The panel layout is this library's one-time weight repack, after the "QTensor and QMatMul" page's
section on the 8-column Q4K repack (blocks of adjacent rows interleaved once on first use, the
original kept): 16 rows x 256 values per panel, codes split from scales.  The layout itself is
pinned by hand-derived single-byte probes (tests/golden/panel_layout_probes.txt) and by a count
that every panel byte is written exactly once; the repack's purpose -- decoding the panels gives
the original values -- by comparing with the original layout's decoder on random weights.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TYPES = [oracle.Q4_K, oracle.Q5_K, oracle.Q6_K, oracle.Q8_0, oracle.Q4_0]
STEP = {oracle.Q4_K: 144, oracle.Q5_K: 176, oracle.Q6_K: 210, oracle.Q8_0: 272, oracle.Q4_0: 144}


def _probes():
    out = []
    with open(os.path.join(GOLDEN, "panel_layout_probes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(tuple(int(t) for t in line.split()))
    return out


@pytest.mark.parametrize("probe", _probes())
def test_panel_probe_lands_where_derived(probe):
    qtype, rows, k, row, step, o, expect = probe
    rb = oracle.row_bytes(qtype, k)
    w = np.zeros(rows * rb, dtype=np.uint8)
    w[row * rb + step * STEP[qtype] + o] = 0xA5
    wp = oracle.repack_panels(qtype, w, rows, k)
    nz = np.flatnonzero(wp)
    assert nz.tolist() == [expect]
    assert wp[expect] == 0xA5


def test_probe_file_covers_every_type():
    assert {p[0] for p in _probes()} == set(TYPES)


@pytest.mark.parametrize("qtype", TYPES)
def test_panel_offsets_are_a_permutation(qtype):
    B = STEP[qtype]
    offs = [oracle.panel_offset(qtype, i, o) for i in range(16) for o in range(B)]
    assert sorted(offs) == list(range(16 * B))


@pytest.mark.parametrize("qtype", TYPES)
def test_panel_bytes(qtype):
    B = STEP[qtype]
    assert oracle.panel_bytes(qtype, 16, 256) == 16 * B
    assert oracle.panel_bytes(qtype, 17, 512) == 2 * 2 * 16 * B          # two groups, two steps
    assert oracle.panel_bytes(qtype, 4096, 4096) == 4096 // 16 * 16 * 16 * B
    assert oracle.panel_bytes(qtype, 4096, 4096) == 4096 * oracle.row_bytes(qtype, 4096)   # same bytes
    assert oracle.panel_bytes(qtype, 16, 96) == -1                        # k not a multiple of 256
    assert oracle.panel_bytes(qtype, 0, 256) == -1
    assert oracle.panel_bytes(3, 16, 256) == -1                           # unsupported type


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("rows", [1, 16, 37])
def test_panels_decode_to_original_values(qtype, rows):
    rng = synth.rngs(300 + qtype + rows, 1)[0]
    k = 768
    w = synth.gen_weights(qtype, rows, k, rng)
    wp = oracle.repack_panels(qtype, w, rows, k)
    assert wp.size == oracle.panel_bytes(qtype, rows, k)
    ref = oracle.dequantize(qtype, w, rows, k)
    got = oracle.dequantize_panels(qtype, wp, rows, k)
    assert np.array_equal(ref, got)
    # the padding rows of the last group are zero bytes
    S, P = k // 256, 16 * STEP[qtype]
    g = (rows - 1) // 16
    for s in range(S):
        panel = wp[(g * S + s) * P:(g * S + s + 1) * P]
        live = {oracle.panel_offset(qtype, i, o) for i in range(rows - 16 * g) for o in range(STEP[qtype])}
        dead = np.array(sorted(set(range(P)) - live), dtype=np.int64)
        assert not panel[dead].any()


def test_decoding_a_wrong_layout_differs():
    """A panel buffer read as if it were the original layout decodes to other values: the pin
    above is not satisfied by an identity repack."""
    rng = synth.rngs(77, 1)[0]
    w = synth.gen_weights(oracle.Q4_K, 16, 512, rng)
    wp = oracle.repack_panels(oracle.Q4_K, w, 16, 512)
    assert not np.array_equal(wp, w.reshape(-1))
    assert not np.array_equal(oracle.dequantize(oracle.Q4_K, wp, 16, 512), oracle.dequantize(oracle.Q4_K, w, 16, 512))
