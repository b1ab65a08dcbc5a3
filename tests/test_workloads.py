"""Seeded workload generators: deterministic, with the stated distributions, and
giving the expected metadata and compression ratios (reduced sizes, CPU only)."""
import numpy as np
import pytest

import oracle
import workloads


def test_deterministic():
    a = workloads.generate("gnn", 0.002)
    b = workloads.generate("gnn", 0.002)
    assert np.array_equal(a.data, b.data) and np.array_equal(a.sample_rows, b.sample_rows)
    assert not np.array_equal(workloads.generate("tiny").data[:100], a.data.reshape(-1)[:100])


def test_distributions():
    g = workloads.generate("gnn", 0.01)
    zero = (g.data == 0).mean()
    assert 0.49 < zero < 0.51 and (g.data >= 0).all()
    assert np.signbit(g.data).sum() == 0  # exact +0.0, never -0.0
    d = workloads.generate("dlrm", 0.001)
    assert d.data.min() >= -0.05 and d.data.max() <= 0.05 and abs(d.data.mean()) < 1e-3
    t = workloads.generate("tiny")
    assert abs(t.data.std() - 0.02) < 5e-4
    ids = workloads.generate("ids", 0.002)
    big = ids.data >= (1 << 24)
    assert 0.045 < big.mean() < 0.055 and ids.data.max() < (1 << 40) and ids.data.min() >= 0
    assert (ids.sample < (1 << 24)).all()  # sampled before the replacement
    llm = workloads.generate("llm", 0.002)
    f = (llm.data.astype(np.uint32) << 16).view(np.float32)
    out = np.abs(f) > 0.01
    assert 0.0005 < out.mean() < 0.002


def test_sample_rows_distinct_and_gather_ids():
    g = workloads.generate("gnn", 0.05)
    rows = g.sample_rows
    assert len(np.unique(rows)) == len(rows) and np.all(np.diff(rows) > 0)
    assert np.array_equal(g.sample, g.data[rows])
    ids = workloads.gather_ids("gnn", g.data.shape[0], 3, 5000)
    assert ids.shape == (3, 5000) and ids.min() >= 0 and ids.max() < g.data.shape[0]
    assert not np.array_equal(ids[0], ids[1])
    z = workloads.gather_ids("dlrm", 100_000, 2, 20000)
    assert z.min() >= 0 and z.max() < 100_000
    _, counts = np.unique(z, return_counts=True)
    assert counts.max() > 200  # the most popular row is hit far more than uniform (0.4)


# expected Mask and stream ratio per workload (hand analysis of each distribution)
EXPECTED = {
    "tiny": (0x78000000, 0x38000000, 1.1033),
    "gnn": (0xC0000000, 0x0, 1.0307),
    "dlrm": (0x7800000078000000, 0x3800000038000000, 1.1226),
    "llm": (0x7C007C007C007C00, 0x3800380038003800, 1.3634),
    "ids": (0xFFFFFFFFFF000000, 0x0, 2.3705),
    # 95% exact zeros: every bit keeps the value 0 in >= 90% of the samples, so a zero
    # chunk costs its participation bit only: 32 / (0.95 * 1 + 0.05 * 33) = 12.31
    "sparse": (0xFFFFFFFF, 0x0, 12.31),
    # the llm tensor one bf16 per chunk: the same exponent bits per element, matched with
    # P = 0.97468, so 16 / (17 - 5 * 0.97468) = 1.3194 (one participation bit per element)
    "llm16": (0x7C00, 0x3800, 1.3194),
    # ids keep their 12 high bits at 0, N(0,1) floats no bit in >= 98% of the rows
    # (|x| < 2 holds for 95.4%), so no bit is invariant across the whole row: every
    # chunk keeps its 64 bits plus its participation bit, 64 / 65
    "mixed": (0x0, 0x0, 0.98462),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_expected_metadata_and_ratio(name):
    inst = workloads.generate(name, {"tiny": 1, "gnn": 0.02, "dlrm": 0.002, "llm": 0.002, "ids": 0.002, "sparse": 0.02,
                                    "llm16": 0.002, "mixed": 0.005}[name])
    W = inst.w.W
    mask, bitval, _ = oracle.build_meta(inst.sample, W, inst.w.T)
    em, eb, er = EXPECTED[name]
    assert (mask, bitval) == (em, eb)
    x = inst.data.reshape(-1)
    off = oracle.offsets(x, W, mask, bitval, inst.w.S)
    ratio = x.nbytes * 8 / int(off[-1])
    assert abs(ratio / er - 1) < 0.01, ratio


def test_mixed_rows_position_metadata():
    """Feature rows (32 ids < 2^20, then 32 N(0,1) floats): the per-position tables
    find each id chunk's 2 x 12 zero bits and nothing in the float chunks, so a row
    of 32 chunks costs 16 (65 - 24) + 16 x 65 = 1696 bits for 2048: ratio 1.2075."""
    inst = workloads.generate("mixed", 0.005)
    ids = inst.data[:, :32]
    dense = inst.data[:, 32:].view(np.float32)
    assert ids.max() < (1 << 20) and ids.max() > (1 << 19)
    assert abs(dense.std() - 1.0) < 0.02 and abs(dense.mean()) < 0.02
    W, S, T = inst.w.W, inst.w.S, inst.w.T
    pm, pb, _ = oracle.build_meta_pos(inst.sample.reshape(-1).view(np.uint8), W, S, T)
    assert (pm[:16] == np.uint64(0xFFF00000FFF00000)).all() and (pm[16:] == 0).all() and (pb == 0).all()
    x = inst.data.reshape(-1)
    off = oracle.offsets_pos(x, W, pm, pb, S)
    assert int(off[-1]) == inst.data.shape[0] * 1696
    assert abs(x.nbytes * 8 / int(off[-1]) - 2048 / 1696) < 1e-12
