"""GPU parity of the position-dependent metadata variant (one Mask/Bitval per chunk
position of a segment) against the oracle, bit-exact: per-position counts, Masks
and Bitvals, offsets, stream bytes and round trips, for W = 16, 32, 64 and the
three segment-size regimes (S dividing 64, S a multiple of 64, any other S)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DT = {16: np.uint16, 32: np.uint32, 64: np.uint64}


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


def say(msg):
    print(msg, flush=True)


def _rand(rng, n, W):
    return (rng.integers(0, 1 << 62, size=n, dtype=np.uint64) * np.uint64(4) +
            rng.integers(0, 4, size=n, dtype=np.uint64)) & np.uint64((1 << W) - 1 if W < 64 else ~0 & (2**64 - 1))


def _tables(rng, S, W):
    """Per-position Masks of every kind: empty, full, one run, alternating bits, random."""
    full = (1 << W) - 1
    kinds = [0, full, ((1 << (W // 2)) - 1) << (W // 4), int("01" * (W // 2), 2), int("0011" * (W // 4), 2)]
    masks = [kinds[i] if i < len(kinds) else int(rng.integers(0, 1 << 62)) & full for i in range(S)]
    rng.shuffle(masks)
    bitvals = [int(rng.integers(0, 1 << 62)) & m for m in masks]
    return np.array(masks, np.uint64), np.array(bitvals, np.uint64)


def _data(rng, n, W, masks, bitvals, S, p=0.7):
    v = _rand(rng, n, W)
    pos = np.arange(n) % S
    hit = rng.random(n) < p
    full = np.uint64((1 << W) - 1) if W < 64 else np.uint64(2**64 - 1)
    v[hit] = (v[hit] & (~masks[pos[hit]] & full)) | bitvals[pos[hit]]
    return v.astype(DT[W])


def _meta(ibp, dev, W, S, masks, bitvals):
    return ibp.PosMeta(W, S, torch.from_numpy(masks.view(np.int64)).to(dev),
                       torch.from_numpy(bitvals.view(np.int64)).to(dev))


@pytest.mark.parametrize("W", [16, 32, 64])
@pytest.mark.parametrize("S", [1, 3, 8, 16, 32, 64, 100, 128, 192, 256, 1000, 1024])
def test_pos_compress_decompress_parity(ibp, W, S):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31 * W + S)
    masks, bitvals = _tables(rng, S, W)
    meta = _meta(ibp, dev, W, S, masks, bitvals)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for n in sorted({1, 63, 64, 65, max(S - 1, 1), S, S + 1, 3 * S + 7, 5000, 70_001}):
        say(f"pos W={W} S={S} n={n}")
        v = _data(rng, n, W, masks, bitvals, S)
        x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
        ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
        nb = ref_stream.size
        # both compression tile forms: the size-chosen one, and the two-half tiles
        # forced on this small input (threshold 0; W = 64 with S a power of two)
        for form, threshold in (("default tiles", 0xFFFFFFFFFFFFFFFF), ("two-half tiles", 0)):
            ibp.ibp_set_halves_min_chunks(threshold)
            try:
                comp = ibp.ibp_compress_pos(meta, x, err=err)
            finally:
                ibp.ibp_set_halves_min_chunks(0xFFFFFFFFFFFFFFFF)
            assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), f"n={n}, {form}: offsets"
            got = comp.stream[:nb].cpu().numpy()
            if not np.array_equal(got, ref_stream):
                bad = int(np.nonzero(got != ref_stream)[0][0])
                raise AssertionError(f"n={n}, {form}: stream differs first at byte {bad} of {nb}")
        out = ibp.ibp_decompress_pos(meta, comp.stream, comp.offsets, n, err=err)
        assert torch.equal(out, x), f"n={n}: round trip"
        s2 = torch.from_numpy(ref_stream.copy()).to(dev)
        out2 = ibp.ibp_decompress_pos(meta, s2, torch.from_numpy(ref_off.view(np.int64)).to(dev), n, err=err)
        assert torch.equal(out2, x), f"n={n}: decode of the oracle stream"
        torch.cuda.synchronize()
        assert int(err.item()) == 0


def _data_rows(rng, n, W, masks, bitvals, S, p):
    """As _data, row by row (fast for large n): chunk j has position j % S."""
    dt = DT[W]
    v = rng.integers(0, np.iinfo(dt).max, size=n, dtype=dt, endpoint=True)
    rows = n // S
    body = v[: rows * S].reshape(rows, S)
    hit = rng.random((rows, S)) < p
    m, b = masks.astype(dt), bitvals.astype(dt)
    body[...] = np.where(hit, (body & ~m[None, :]) | b[None, :], body)
    return v


# n above what four times the resident workgroups cover in one sweep (the grid is
# capped there and each workgroup loops over tiles), for the paths: W = 16 pairs
# with shift steps, W = 32 any S, W = 64 one chunk per lane; the smaller cases add
# the W = 16 one-per-lane and W = 32 pair paths, a W = 64 S of one tile per wave, and
# W = 64 with S dividing 64 (whole segments per pass; the ragged last tile takes the
# general path).
@pytest.mark.parametrize("W,S,n", [(16, 1024, (1 << 25) + 77), (32, 100, 20_000_077), (64, 256, (1 << 24) + 77),
                                   (16, 64, 1_000_077), (32, 256, 1_000_077), (64, 1000, 1_000_077),
                                   (64, 32, 2_000_077)])
def test_pos_decode_many_tiles(ibp, W, S, n):
    """Large inputs (each workgroup loops over many tiles): the decode of the
    oracle's stream equals the input, and so do decodes into outputs one and two
    chunks past an 8-byte boundary (W = 16 stores four chunks per lane as one
    word only from 8-byte aligned outputs, two from 4-byte aligned ones)."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5 * W + S)
    masks, bitvals = _tables(rng, S, W)
    meta = _meta(ibp, dev, W, S, masks, bitvals)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"pos many tiles W={W} S={S} n={n}")
    v = _data_rows(rng, n, W, masks, bitvals, S, 0.8)
    ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
    x = torch.from_numpy(v.view(np.uint8)).to(dev)
    s_d = torch.from_numpy(ref_stream).to(dev)
    o_d = torch.from_numpy(ref_off.view(np.int64)).to(dev)
    out = ibp.ibp_decompress_pos(meta, s_d, o_d, n, err=err)
    assert torch.equal(out, x), "decode of the oracle stream"
    del out
    cb = W // 8
    big = torch.zeros(n * cb + 16, dtype=torch.uint8, device=dev)
    for k in (1, 2):  # one and two chunks past an 8-byte boundary (the narrower store forms)
        out2 = big[k * cb: k * cb + n * cb]
        out2.zero_()
        ibp.ibp_decompress_pos(meta, s_d, o_d, n, out=out2, err=err)
        assert torch.equal(out2, x), f"decode into an output {k} chunk(s) past alignment"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("W", [16, 32, 64])
@pytest.mark.parametrize("S", [1, 5, 128, 1000])
def test_pos_metadata_parity(ibp, W, S):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7 * W + S)
    R = 3001
    base = _rand(rng, R * S, W).reshape(R, S)
    bias = _rand(rng, S, W)
    keep = rng.random((R, S)) < 0.93
    rows = np.where(keep, base & bias, base).astype(DT[W])
    x = torch.from_numpy(rows.reshape(-1).view(np.uint8).copy()).to(dev)
    for T in (0.51, 0.9, 0.95, 1.0):
        say(f"pos metadata W={W} S={S} T={T}")
        meta, counts = ibp.ibp_build_metadata_pos(x, W, S, T)
        masks, bitvals, c1 = oracle.build_meta_pos(rows.reshape(-1), W, S, T)
        assert np.array_equal(np.array(counts, np.uint64), c1)
        assert np.array_equal(meta.mask.cpu().numpy().view(np.uint64), masks)
        assert np.array_equal(meta.bitval.cpu().numpy().view(np.uint64), bitvals)


def test_pos_tables_are_sanitised(ibp):
    """Bits of Mask_i at or above W and bits of Bitval_i outside Mask_i are ignored:
    the result equals the oracle run on the cleaned tables."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(3)
    W, S, n = 32, 64, 20_000
    masks, bitvals = _tables(rng, S, W)
    v = _data(rng, n, W, masks, bitvals, S)
    dirty_m = masks | np.uint64(0xFFFF_0000_0000_0000)
    dirty_b = bitvals | (~masks & np.uint64(0xFFFF_FFFF))
    meta = _meta(ibp, dev, W, S, dirty_m, dirty_b)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    comp = ibp.ibp_compress_pos(meta, x)
    ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
    assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off)
    assert np.array_equal(comp.stream[:ref_stream.size].cpu().numpy(), ref_stream)
    assert torch.equal(ibp.ibp_decompress_pos(meta, comp.stream, comp.offsets, n), x)


def test_pos_corrupt_offsets_reported(ibp):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(4)
    W, S, n = 32, 128, 50_000
    masks, bitvals = _tables(rng, S, W)
    v = _data(rng, n, W, masks, bitvals, S)
    ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
    bad = ref_off.copy()
    bad[10] += 3  # segment 9 too long, segment 10 too short
    meta = _meta(ibp, dev, W, S, masks, bitvals)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = ibp.ibp_decompress_pos(meta, torch.from_numpy(ref_stream.copy()).to(dev),
                                 torch.from_numpy(bad.view(np.int64)).to(dev), n, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
    got = out.cpu().numpy().view(np.uint32).reshape(-1)
    # segments far from the damaged ones still decode
    assert np.array_equal(got[:9 * S], v[:9 * S]) and np.array_equal(got[12 * S:], v[12 * S:])
