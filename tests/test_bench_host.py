"""Host-side pieces of bench.py that decide reported figures, on the CPU.

The N-thread oracle baseline compresses segment ranges into private buffers and
joins them at bit level (``bench._stitch``); its result must equal the oracle's
one-piece stream of the same segments (1 thread == N threads), for part lengths that
are not multiples of 8 bits and with more parts than threads."""
import numpy as np
import pytest

import bench
import oracle


def _encode_ranges(v, W, mask, bitval, S, ranges):
    parts, offs, base = [], [np.zeros(1, np.uint64)], 0
    for k0, k1 in ranges:
        seg = v[k0 * S: min(k1 * S, v.size)]
        buf, off = oracle.encode(seg, W, mask, bitval, S)
        nb = int(off[-1])
        parts.append((np.concatenate([buf, np.zeros(1, np.uint8)]), nb))
        offs.append(off[1:] + np.uint64(base))
        base += nb
    return parts, np.concatenate(offs), base


@pytest.mark.parametrize("W,S,parts", [(32, 7, 5), (64, 3, 13), (16, 100, 4), (32, 1, 64), (64, 256, 3)])
def test_stitched_ranges_equal_one_piece(W, S, parts):
    rng = np.random.default_rng(W * 31 + S * 7 + parts)
    n = int(rng.integers(S * parts, S * parts * 20))
    full = (1 << W) - 1
    mask = int(rng.integers(0, 1 << 32)) & full
    bitval = int(rng.integers(0, 1 << 32)) & mask
    v = rng.integers(0, 1 << 63, n, dtype=np.uint64) & np.uint64(full)
    keep = rng.random(n) < 0.7
    v[keep] = (v[keep] & ~np.uint64(mask)) | np.uint64(bitval)
    v = v.astype({16: np.uint16, 32: np.uint32, 64: np.uint64}[W])
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    nseg = (n + S - 1) // S
    pieces, off, total = _encode_ranges(v, W, mask, bitval, S, bench._ranges(nseg, parts))
    assert total == int(ref_off[-1])
    assert np.array_equal(off, ref_off)
    for threads in (1, 4):
        got = bench._stitch(pieces, total, threads)
        assert np.array_equal(got, ref_stream), f"{threads} threads"


def test_ranges_cover_every_segment_once():
    for n, p in ((1, 4), (10, 3), (1000, 7), (5, 5), (3, 8)):
        r = bench._ranges(n, p)
        assert r[0][0] == 0 and r[-1][1] == n
        assert all(a < b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
