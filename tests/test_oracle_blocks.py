"""Pins of the oracle's blocking, packing and 2-D views (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_dash_blocking_worked_example():
    g = _golden("dash_blocking_example.json")
    t = oracle.plan_blocks([(g["V"], g["E"])], [g["B"]])
    rows, cols = t[:, 5], t[:, 6]
    full = (rows == g["B"]) & (cols == g["B"])
    assert full.sum() == g["G_full"][0]
    rest = ~full
    assert rest.sum() == g["G_rest"][0]
    assert set(zip(rows[rest], cols[rest])) == {tuple(g["G_rest"][1:])}
    # factor shapes: L of a block is rows x rows, R is cols x cols
    sides = np.concatenate([rows, cols])
    assert (sides == g["S_full"][1]).sum() == g["S_full"][0]
    assert (sides == g["S_rest"][1]).sum() == g["S_rest"][0]


def test_dash_reshape_example():
    g = _golden("dash_reshape_example.json")
    assert oracle.reshape_2d(g["shape"]) == tuple(g["view2d"])
    assert oracle.reshape_2d((7,)) == (1, 7)
    assert oracle.reshape_2d(()) == (1, 1)


def test_table_order_and_offsets():
    shapes = [(300, 130), (64, 64), (5, 700)]
    t = oracle.plan_blocks(shapes, [128, 128, 256])
    # parameter by parameter, row-major over the block grid
    expect = []
    for p, ((m, n), B) in enumerate(zip(shapes, [128, 128, 256])):
        for br in range((m + B - 1) // B):
            for bc in range((n + B - 1) // B):
                expect.append((p, br, bc, br * B, bc * B, min(B, m - br * B), min(B, n - bc * B), B))
    assert [tuple(int(x) for x in r) for r in t] == expect
    # blocks tile every parameter exactly once
    for p, (m, n) in enumerate(shapes):
        cover = np.zeros((m, n), dtype=int)
        for b in np.nonzero(t[:, 0] == p)[0]:
            rs, cs = oracle.block_slices(t, b)
            cover[rs, cs] += 1
        assert (cover == 1).all()


def test_block_size_not_smaller_than_param_gives_one_padded_block():
    t = oracle.plan_blocks([(40, 70)], [128])
    assert t.shape == (1, 8)
    assert tuple(t[0]) == (0, 0, 0, 0, 0, 40, 70, 128)
    t0 = oracle.plan_blocks([(40, 70)], [0])
    assert tuple(t0[0]) == (0, 0, 0, 0, 0, 40, 70, 70)


def test_pack_unpack_elementwise():
    gen = np.random.default_rng(1)
    shapes = [(300, 130), (64, 64)]
    mats = [gen.standard_normal(s) for s in shapes]
    B = 128
    t = oracle.plan_blocks(shapes, [B, B])
    st = oracle.pack_blocks(mats, t, B)
    assert st.shape == (t.shape[0], B, B)
    for b in range(t.shape[0]):
        p, _, _, r0, c0, rows, cols, _ = (int(x) for x in t[b])
        for i in range(B):
            for j in range(0, B, 17):
                want = mats[p][r0 + i, c0 + j] if (i < rows and j < cols) else 0.0
                assert st[b, i, j] == want
    back = oracle.unpack_blocks(st, t, shapes)
    for a, b in zip(mats, back):
        assert np.array_equal(a, b)


def test_workload_shapes():
    sh4 = synthetic.decoder_shapes()
    assert len(sh4) == 48 and sum(m * n for m, n in sh4) == 150994944
    t4 = oracle.plan_blocks(sh4, [1024] * 48)
    assert t4.shape[0] == 144 and (t4[:, 5] == 1024).all() and (t4[:, 6] == 1024).all()
    sh5 = synthetic.bottleneck50_shapes()
    bs5 = synthetic.bottleneck50_block_sizes(sh5)
    assert len(sh5) == 53 and sum(m * n for m, n in sh5) == 25493504
    t5 = oracle.plan_blocks(sh5, bs5)
    assert (t5[:, 7] == 256).sum() == 115 and (t5[:, 7] == 1024).sum() == 47
