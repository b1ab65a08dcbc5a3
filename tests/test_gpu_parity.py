"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit-exact.

Tolerance is 0 everywhere: the codec is lossless, so counts, Mask, Bitval, the
offset table, every stream byte below ceil(total/8) and the round trip must
agree exactly.  Sizes span several compression tiles (8,192 or 16,384 chunks,
4,096 with position metadata) and decompression tiles (512 chunks per wavefront)
plus ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DT = {16: np.uint16, 32: np.uint32, 64: np.uint64}
# an exponent-like Mask and its Bitval per width, for the gather and slot tests
GMASK = {16: (0x7800, 0x3800), 32: (0xC0000000, 0), 64: (0x7800000078000000, 0x3800000038000000)}


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


def say(msg):
    print(msg, flush=True)


def _data(rng, n, W, mask, bitval, p_match):
    """n W-bit chunks: random free bits; invariant bits equal Bitval with probability p_match."""
    if W == 16:
        v = rng.integers(0, 1 << 16, size=n, dtype=np.uint64).astype(np.uint16)
    elif W == 32:
        v = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    else:
        v = rng.integers(0, 1 << 63, size=n, dtype=np.uint64) * np.uint64(2) + \
            rng.integers(0, 2, size=n, dtype=np.uint64)
    t = DT[W]
    keep = rng.random(n) < p_match
    v[keep] = (v[keep] & t(~mask & ((1 << W) - 1))) | t(bitval)
    return v


def _masks(rng, W):
    full = (1 << W) - 1
    exp = {16: 0x7C00, 32: 0x78000000, 64: 0x7C007C007C007C00}[W]
    m = int(rng.integers(0, 1 << 62)) & full
    return [
        ("zero", 0, 0),
        ("full", full, int(rng.integers(0, 1 << 62)) & full),
        ("exponent", exp, exp & 0x3838383838383838),
        ("random", m, int(rng.integers(0, 1 << 62)) & m),
    ]


def _run_case(ibp, dev, v, W, S, mask, bitval, tag):
    n = v.size
    say(f"case {tag}: W={W} S={S} n={n} mask={mask:#x}")
    meta = ibp.make_meta(W, mask, bitval)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    nb = (int(ref_off[-1]) + 7) // 8
    # both compression tile forms: the size-chosen one, and the large two-half tiles
    # forced on this small input (threshold 0)
    for form, threshold in (("default tiles", 0xFFFFFFFFFFFFFFFF), ("two-half tiles", 0)):
        ibp.ibp_set_halves_min_chunks(threshold)
        try:
            comp = ibp.ibp_compress(meta, x, S, err=err)
        finally:
            ibp.ibp_set_halves_min_chunks(0xFFFFFFFFFFFFFFFF)
        off = comp.offsets.cpu().numpy().view(np.uint64)
        assert np.array_equal(off, ref_off), f"{tag}, {form}: offsets differ"
        got = comp.stream[:nb].cpu().numpy()
        if not np.array_equal(got, ref_stream):
            bad = int(np.nonzero(got != ref_stream)[0][0])
            raise AssertionError(f"{tag}, {form}: stream differs first at byte {bad} of {nb}")
    # decode the GPU stream
    out = ibp.ibp_decompress(meta, comp.stream, comp.offsets, n, S, err=err)
    assert torch.equal(out, x), f"{tag}: round trip differs"
    # decode the oracle stream from an exactly sized buffer (tail block read byte-wise)
    if nb:
        s2 = torch.from_numpy(ref_stream.copy()).to(dev)
        out2 = ibp.ibp_decompress(meta, s2, torch.from_numpy(ref_off.view(np.int64)).to(dev), n, S, err=err)
        assert torch.equal(out2, x), f"{tag}: decode of the oracle stream differs"
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f"{tag}: device error word {int(err.item())}"


@pytest.mark.parametrize("W", [16, 32, 64])
@pytest.mark.parametrize("S", [1, 3, 32, 64, 100, 128, 192, 256, 1000, 1024])
def test_compress_decompress_parity(ibp, W, S):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(W * 10007 + S)
    sizes = sorted({0, 1, 63, 64, 65, max(S - 1, 1), S, S + 1, 3 * S + 7, 5000, 70_001})
    for name, mask, bitval in _masks(rng, W):
        for n in sizes:
            p = 0.9 if name != "zero" else 1.0
            _run_case(ibp, dev, _data(rng, n, W, mask, bitval, p), W, S, mask, bitval, f"{name}-{n}")


@pytest.mark.parametrize("W", [32, 64])
@pytest.mark.parametrize("S", [1, 32, 64, 256])
def test_tiles_near_the_half_image_size(ibp, W, S):
    """One Mask and S a power of two: a compression tile whose stream size is at
    most that of half the tile stored raw is packed whole and stored once, a larger
    one in two halves.  The tile is 16,384 chunks here for both widths (W = 32; and
    W = 64 with more than 32 invariant bits, where a tile can fit at all), forced on
    this small input by the case runner, which compresses with both tile forms.  Tiles
    alternate between the two forms, including sizes exactly at the limit and one
    chunk's saving on either side of it, and end in a ragged tail; every byte must
    match the oracle."""
    dev = torch.device("cuda:0")
    tile = 16384
    pc = 24 if W == 32 else 40  # popcount(Mask); tile (W + 1) / (2 pc) is an integer
    mask = ((1 << pc) - 1) << (W - pc)
    bitval = mask & 0x5A5A5A5A5A5A5A5A
    limit = tile * (W + 1) // 2      # the largest tile that is packed whole, in bits
    k_at = (tile * (W + 1) - limit) // pc  # matching chunks that give exactly that size
    rng = np.random.default_rng(W * 7 + S)
    # matching chunks per tile: exactly at the limit, one saving short of it, none,
    # all, and random fractions; then a ragged tail
    counts = [k_at, k_at - 1, 0, tile, k_at + 1, tile // 3]
    parts = []
    for k in counts:
        v = _data(rng, tile, W, mask, bitval, 0.0)
        keep = rng.permutation(tile)[:k]
        t = DT[W]
        v[keep] = (v[keep] & t(~mask & ((1 << W) - 1))) | t(bitval)
        # no chunk outside `keep` may match by chance
        others = np.setdiff1d(np.arange(tile), keep)
        hit = ((v[others] ^ t(bitval)) & t(mask)) == 0
        v[others[hit]] ^= t(1 << (W - 1))
        parts.append(v)
    parts.append(_data(rng, 3 * tile // 4 + 5, W, mask, bitval, 0.5))
    v = np.concatenate(parts)
    _run_case(ibp, dev, v, W, S, mask, bitval, f"half-image W={W} S={S}")


@pytest.mark.parametrize("W", [16, 32])
@pytest.mark.parametrize("S", [128, 256])
def test_decode_into_unaligned_output(ibp, W, S):
    """Outputs that start one or two chunks past an 8-byte boundary: the decoders
    store four W = 16 chunks or a pair of W <= 32 chunks as one word only when the
    output allows it, else fewer chunks per lane; the contiguous decode (both
    offsets) and the HBM gather (one chunk) are checked."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(W * 31 + S)
    cb = W // 8
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for name, mask, bitval in _masks(rng, W):
        for n in (20 * S, 20 * S + 5):
            say(f"unaligned output {name} W={W} S={S} n={n}")
            v = _data(rng, n, W, mask, bitval, 0.9)
            meta = ibp.make_meta(W, mask, bitval)
            x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
            comp = ibp.ibp_compress(meta, x, S, err=err)
            big = torch.zeros(n * cb + 16, dtype=torch.uint8, device=dev)
            for k in (1, 2):  # one and two chunks past an 8-byte boundary
                out = big[k * cb: k * cb + n * cb]
                out.zero_()
                ibp.ibp_decompress(meta, comp.stream, comp.offsets, n, S, out=out, err=err)
                assert torch.equal(out, x), f"{name} n={n}: contiguous decode {k} chunk(s) past alignment"
            ids_np = rng.integers(0, n // S, 300).astype(np.int64)
            big2 = torch.zeros(ids_np.size * S * cb + 16, dtype=torch.uint8, device=dev)
            out2 = big2[cb: cb + ids_np.size * S * cb]
            ibp.ibp_decompress_gather(meta, comp.stream, comp.offsets, S, torch.from_numpy(ids_np).to(dev),
                                      out=out2, err=err, n_segments=n // S)
            want = v[: (n // S) * S].reshape(-1, S)[ids_np].reshape(-1)
            assert np.array_equal(out2.cpu().numpy().view(v.dtype), want), f"{name} n={n}: gather into an unaligned output"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("W", [16, 32, 64])
def test_all_invariant_and_raw_streams(ibp, W):
    """Minimum size (all chunks equal Bitval on a full Mask) and +1 bit per chunk (Mask = 0)."""
    dev = torch.device("cuda:0")
    full = (1 << W) - 1
    v = np.zeros(40_000, DT[W])
    _run_case(ibp, dev, v, W, 256, full, 0, "all-invariant")
    rng = np.random.default_rng(9)
    _run_case(ibp, dev, _data(rng, 40_000, W, 0, 0, 0.0), W, 256, 0, 0, "raw")


@pytest.mark.parametrize("W", [16, 32, 64])
@pytest.mark.parametrize("T", [0.51, 0.9, 0.99, 1.0])
def test_metadata_parity(ibp, W, T):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(int(T * 1000) + W)
    for n in (1, 2, 255, 4096, 100_003, 1_500_000):
        base = _data(rng, n, W, 0, 0, 0.0)
        # bias the bits so that several positions sit near the threshold
        bias = DT[W](rng.integers(0, 1 << min(W - 1, 62)))
        v = np.where(rng.random(n) < T, base & bias, base)
        say(f"metadata W={W} T={T} n={n}")
        meta, counts = ibp.ibp_build_metadata(torch.from_numpy(v.view(np.uint8).copy()).to(dev), W, T)
        mask, bitval, c1 = oracle.build_meta(v, W, T)
        assert counts == c1.tolist()
        assert (meta.mask, meta.bitval, meta.W) == (mask, bitval, W)


@pytest.mark.parametrize("W,S", [(32, 128), (64, 32), (64, 1), (32, 1000), (16, 128), (16, 40), (16, 512)])
@pytest.mark.parametrize("where", ["device", "pinned"])
def test_gather_parity(ibp, W, S, where):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(S + W)
    nseg = 3000
    mask, bitval = GMASK[W]
    v = _data(rng, nseg * S, W, mask, bitval, 0.95)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    meta = ibp.make_meta(W, mask, bitval)
    if where == "device":
        src = torch.from_numpy(ref_stream.copy()).to(dev)
    else:
        src = torch.empty(ref_stream.size, dtype=torch.uint8, pin_memory=True)
        src.copy_(torch.from_numpy(ref_stream))
    off = torch.from_numpy(ref_off.view(np.int64)).to(dev)
    ids_np = rng.integers(0, nseg, size=4099).astype(np.int64)
    ids_np[:3] = [0, nseg - 1, 0]  # first, last, duplicate
    ids = torch.from_numpy(ids_np).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"gather W={W} S={S} from {where}")
    rows = ibp.ibp_decompress_gather(meta, src, off, S, ids, err=err)
    ref = oracle.decode_gather(ref_stream, ref_off, S, ids_np, W, mask, bitval, np.uint8)
    assert np.array_equal(rows.cpu().numpy(), ref)
    assert np.array_equal(ref.view(DT[W]).reshape(len(ids_np), S), v.reshape(nseg, S)[ids_np])
    assert int(err.item()) == 0


@pytest.mark.parametrize("W,S", [(32, 128), (64, 32), (32, 100), (64, 1), (32, 256), (16, 256), (64, 64), (32, 64),
                                 (16, 128)])
def test_gather_many_ids(ibp, W, S):
    """A gather from HBM large enough that several rounds of wavefronts run (and,
    for S >= 64, the per-row staging path, whose rows are decoded four at a time:
    four chunks per lane at W = 16 and S = 256, two at S = 128 and at W = 32 and
    S = 256, one at S = 64);
    compared with the rows themselves and, for a prefix, with the oracle's decode
    of the same stream."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1000 + S + W)
    nseg = 5000
    mask, bitval = GMASK[W]
    v = _data(rng, nseg * S, W, mask, bitval, 0.9)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    meta = ibp.make_meta(W, mask, bitval)
    src = torch.from_numpy(ref_stream.copy()).to(dev)
    off = torch.from_numpy(ref_off.view(np.int64)).to(dev)
    n_ids = max(400_000 // S, 50_000) * 4 + 13
    ids_np = rng.integers(0, nseg, size=n_ids).astype(np.int64)
    ids = torch.from_numpy(ids_np).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"gather W={W} S={S} ids={n_ids}")
    rows = ibp.ibp_decompress_gather(meta, src, off, S, ids, err=err)
    got = rows.cpu().numpy().view(DT[W]).reshape(n_ids, S)
    assert np.array_equal(got, v.reshape(nseg, S)[ids_np])
    ref = oracle.decode_gather(ref_stream, ref_off, S, ids_np[:2048], W, mask, bitval, np.uint8)
    assert np.array_equal(rows[:ref.size].cpu().numpy(), ref)
    assert int(err.item()) == 0


def test_raw_gather(ibp):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1)
    table = rng.integers(0, 255, size=(1000, 512), dtype=np.uint8)
    src = torch.empty(table.size, dtype=torch.uint8, pin_memory=True)
    src.copy_(torch.from_numpy(table.reshape(-1)))
    ids_np = rng.integers(0, 1000, size=777).astype(np.int64)
    say("raw gather from pinned memory")
    out = ibp.ibp_gather_raw(src, 512, torch.from_numpy(ids_np).to(dev))
    assert np.array_equal(out.cpu().numpy().reshape(777, 512), table[ids_np])


def test_device_error_reporting(ibp):
    """Corrupt offsets and bad ids are reported in the error word; nothing is read
    outside the stream and rows with bad ids are left untouched."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(2)
    W, S, mask, bitval = 32, 128, 0xC0000000, 0
    v = _data(rng, 100 * S, W, mask, bitval, 0.9)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    meta = ibp.make_meta(W, mask, bitval)
    stream = torch.from_numpy(ref_stream.copy()).to(dev)
    say("error paths: corrupt offset")
    bad_off = ref_off.copy().view(np.int64)
    bad_off[7] += 3
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ibp.ibp_decompress(meta, stream, torch.from_numpy(bad_off).to(dev), v.size, S, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
    say("error paths: offset past the stream end")
    bad_off = ref_off.copy().view(np.int64)
    bad_off[-1] = (ref_stream.size + 64) * 8
    err.zero_()
    ibp.ibp_decompress(meta, stream, torch.from_numpy(bad_off).to(dev), v.size, S, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
    say("error paths: bad gather ids")
    err.zero_()
    ids = torch.tensor([5, -1, 100, 99], dtype=torch.int64, device=dev)
    out = torch.full((4 * S * 4,), 0xAB, dtype=torch.uint8, device=dev)
    ibp.ibp_decompress_gather(meta, stream, torch.from_numpy(ref_off.view(np.int64)).to(dev), S, ids, out=out,
                              err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ibp.IBP_DEVERR_BAD_ID
    o = out.cpu().numpy().reshape(4, -1)
    assert (o[1] == 0xAB).all() and (o[2] == 0xAB).all()
    assert np.array_equal(o[0].view(np.uint32), v.reshape(100, S)[5])
    assert np.array_equal(o[3].view(np.uint32), v.reshape(100, S)[99])


def test_host_argument_checks(ibp):
    """Pointers the kernels cannot reach are refused before any launch."""
    dev = torch.device("cuda:0")
    meta = ibp.make_meta(32, 0xC0000000, 0)
    pageable = torch.zeros(4096, dtype=torch.uint8)  # ordinary host memory
    off = torch.zeros(2, dtype=torch.int64, device=dev)
    with pytest.raises(ibp.IBPError) as e:
        ibp.ibp_decompress(meta, pageable, off, 128, 128)
    assert e.value.status == ibp.IBP_ERR_INVALID_ARG
    stream = torch.zeros(4096, dtype=torch.uint8, device=dev)
    lib = ibp.load_library()
    # a stream length far beyond the allocation
    rc = lib.ibp_decompress(ibp.ctypes.byref(meta), stream.data_ptr(), 1 << 40, off.data_ptr(), 128, 128,
                            torch.empty(512, dtype=torch.uint8, device=dev).data_ptr(), None, None)
    assert rc == ibp.IBP_ERR_INVALID_ARG


@pytest.mark.parametrize("S", [64, 128])
def test_compress_w16_input_two_bytes_past_alignment(ibp, S):
    """W = 16 input that starts 2 bytes past a 4-byte boundary (the compressor reads
    chunk pairs as 32-bit words only from 4-byte aligned inputs): the same stream
    and offsets as the oracle, and as the compression of an aligned copy."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(S + 16)
    W = 16
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for name, mask, bitval in _masks(rng, W):
        n = 20_000 * (S // 64) + 7
        say(f"w16 input +2 bytes {name} S={S} n={n}")
        v = _data(rng, n, W, mask, bitval, 0.9)
        meta = ibp.make_meta(W, mask, bitval)
        big = torch.zeros(2 * n + 8, dtype=torch.uint8, device=dev)
        x = big[2: 2 + 2 * n]
        x.copy_(torch.from_numpy(v.view(np.uint8).copy()).to(dev))
        comp = ibp.ibp_compress(meta, x, S, err=err)
        ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
        assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), f"{name}: offsets"
        assert np.array_equal(comp.stream[: ref_stream.size].cpu().numpy(), ref_stream), f"{name}: stream"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("src,dst", [("pinned", "device"), ("device", "pinned"), ("pinned", "pinned")])
def test_zero_copy_compress(ibp, src, dst):
    """Compression reading its input from, or writing its stream into, pinned host
    memory through the device mapping (no staging copy): same bytes as the oracle."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(12)
    W, S, mask, bitval = 32, 128, 0x78000000, 0x38000000
    v = _data(rng, 3000 * S + 17, W, mask, bitval, 0.97)
    meta = ibp.make_meta(W, mask, bitval)
    xb = torch.from_numpy(v.view(np.uint8).copy())
    x = xb.to(dev) if src == "device" else xb.pin_memory()
    cap = ibp.ibp_max_stream_bytes(v.size, W)
    out = torch.empty(cap, dtype=torch.uint8, device=dev) if dst == "device" else \
        torch.empty(cap, dtype=torch.uint8, pin_memory=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"zero-copy compress {src} -> {dst}")
    comp = ibp.ibp_compress(meta, x, S, err=err, out_stream=out)
    torch.cuda.synchronize()
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off)
    assert np.array_equal(out[: ref_stream.size].cpu().numpy(), ref_stream)
    back = ibp.ibp_decompress(meta, out, comp.offsets, v.size, S, err=err)
    assert np.array_equal(back.cpu().numpy(), v.view(np.uint8))
    assert int(err.item()) == 0


@pytest.mark.parametrize("W,S", [(64, 256), (16, 1024), (32, 100), (64, 3)])
def test_pinned_stream_decompress(ibp, W, S):
    """Whole-tensor decompression with the oracle's stream in pinned host memory, read
    zero-copy by the decoder (offsets in HBM): the output equals the input, over many
    tiles and a ragged last segment."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(W * 3 + S)
    mask = {16: 0x7C00, 32: 0x78000000, 64: 0x7C007C007C007C00}[W]
    bitval = mask & 0x3838383838383838
    n = 400 * S + S // 2 + 1
    v = _data(rng, n, W, mask, bitval, 0.95)
    meta = ibp.make_meta(W, mask, bitval)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    host = torch.zeros(ibp.ibp_stream_bytes(int(ref_off[-1])), dtype=torch.uint8, pin_memory=True)
    host[: ref_stream.size].copy_(torch.from_numpy(ref_stream))
    off = torch.from_numpy(ref_off.view(np.int64).copy()).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"pinned stream decompress W={W} S={S} n={n}")
    back = ibp.ibp_decompress(meta, host, off, n, S, err=err)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), v.view(np.uint8))
    assert int(err.item()) == 0


@pytest.mark.parametrize("W,S", [(32, 128), (64, 32), (32, 100), (64, 1024), (32, 4), (16, 64), (16, 200)])
@pytest.mark.parametrize("where", ["device", "pinned"])
def test_slots_parity(ibp, W, S, where):
    """Fixed-slot layout: flags and the used prefix of every slot equal the oracle's;
    gathers from device or pinned host slots equal the input rows."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(W * 7 + S)
    R = 1500 if S < 1024 else 300
    mask = {16: 0x7C00, 32: 0x78000000, 64: 0x7C007C007C007C00}[W]
    bitval = mask & 0x3838383838383838
    rows = [_data(rng, S, W, mask, bitval, 0.97 if r % 5 else 0.02) for r in range(R)]
    v = np.concatenate(rows)
    meta = ibp.make_meta(W, mask, bitval)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    row_bytes = S * W // 8
    slots = torch.zeros(R * row_bytes, dtype=torch.uint8, device=dev) if where == "device" else \
        torch.zeros(R * row_bytes, dtype=torch.uint8, pin_memory=True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say(f"slots W={W} S={S} in {where}")
    slots, flags = ibp.ibp_compress_slots(meta, x, S, slots=slots, err=err)
    torch.cuda.synchronize()
    ref_slots, ref_flags, used = oracle.encode_slots(v, W, mask, bitval, S)
    got_flags = flags.cpu().numpy().view(np.uint64)
    assert np.array_equal(got_flags, ref_flags)
    got = slots.cpu().numpy().reshape(R, row_bytes)
    ref = ref_slots.reshape(R, row_bytes)
    for r in range(R):
        nb = (int(used[r]) + 7) // 8
        assert np.array_equal(got[r, :nb], ref[r, :nb]), f"slot {r} differs"
    ids_np = rng.integers(0, R, size=2049).astype(np.int64)
    ids_np[:2] = [0, R - 1]
    out = ibp.ibp_decompress_gather_slots(meta, slots, flags, S, torch.from_numpy(ids_np).to(dev), err=err)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(DT[W]).reshape(len(ids_np), S), v.reshape(R, S)[ids_np])
    assert int(err.item()) == 0


def test_graph_replay(ibp):
    """Compress, decompress and three gathers captured in one HIP graph.  Each of
    several replays, with eager work, fills and synchronisations between them, must
    reproduce the oracle's stream, offsets, round trip and gathered rows."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    W, S, nseg = 32, 128, 2000
    mask, bitval = 0xC0000000, 0
    v = _data(rng, nseg * S, W, mask, bitval, 0.95)
    n = v.size
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    nb = ref_stream.size
    meta = ibp.make_meta(W, mask, bitval)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    stream_g = torch.empty(ibp.ibp_max_stream_bytes(n, W), dtype=torch.uint8, device=dev)
    off_g = torch.empty(nseg + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(ibp.ibp_compress_workspace_bytes(n, S), dtype=torch.uint8, device=dev)
    out_full = torch.empty_like(x)
    ids_np = [rng.integers(0, nseg, size=m).astype(np.int64) for m in (1000, 4096, 77)]
    ids = [torch.from_numpy(i).to(dev) for i in ids_np]
    rows = [torch.empty(i.size * S * 4, dtype=torch.uint8, device=dev) for i in ids_np]
    ref_rows = [oracle.decode_gather(ref_stream, ref_off, S, i, W, mask, bitval, np.uint8) for i in ids_np]

    def work():
        ibp.ibp_compress(meta, x, S, err=err, out_stream=stream_g, out_offsets=off_g, workspace=ws)
        ibp.ibp_decompress(meta, stream_g, off_g, n, S, out=out_full, err=err)
        for i, r in zip(ids, rows):
            ibp.ibp_decompress_gather(meta, stream_g, off_g, S, i, out=r, err=err)

    work()  # eager once before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    other = torch.empty_like(out_full)
    for rep in range(4):
        say(f"graph replay {rep}")
        for t in (stream_g, off_g, out_full, *rows):
            t.zero_()
        ibp.ibp_decompress(meta, torch.from_numpy(ref_stream.copy()).to(dev),
                           torch.from_numpy(ref_off.view(np.int64)).to(dev), n, S, out=other, err=err)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(off_g.cpu().numpy().view(np.uint64), ref_off), f"replay {rep}: offsets"
        assert np.array_equal(stream_g[:nb].cpu().numpy(), ref_stream), f"replay {rep}: stream"
        assert torch.equal(out_full, x), f"replay {rep}: round trip"
        for k, (r, ref) in enumerate(zip(rows, ref_rows)):
            assert np.array_equal(r.cpu().numpy(), ref), f"replay {rep}: gather {k}"
        assert torch.equal(other, x)
    assert int(err.item()) == 0


def test_lookback_give_up_path(ibp):
    """The compressors' bounded wait, forced from the host: with a wait limit of 0 a
    tile that finds an unpublished predecessor gives up at once (no kernel waits).
    A call then either produced the exact stream (no tile had to wait) or reports
    IBP_DEVERR_TIMEOUT, left ~0 in the offsets of the tiles that gave up, and every
    decoder refuses the result.  The default limit is restored afterwards and the
    next compression is exact."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77)
    W, S, mask, bitval = 32, 128, 0xC0000000, 0
    v = _data(rng, 2_000_000, W, mask, bitval, 0.97)
    meta = ibp.make_meta(W, mask, bitval)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    nb = (int(ref_off[-1]) + 7) // 8
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    gave_up = 0
    try:
        ibp.ibp_set_wait_limit(0)
        for it in range(4):
            say(f"give-up path: IBP compression, wait limit 0, call {it}")
            err.zero_()
            comp = ibp.ibp_compress(meta, x, S, err=err)
            torch.cuda.synchronize()
            e = int(err.item())
            off = comp.offsets.cpu().numpy()
            if e == 0:
                assert np.array_equal(off.view(np.uint64), ref_off)
                assert np.array_equal(comp.stream[:nb].cpu().numpy(), ref_stream)
                continue
            gave_up += 1
            assert e == ibp.IBP_DEVERR_TIMEOUT, e
            assert (off == -1).any(), "a tile that gave up leaves ~0 offsets"
            err.zero_()
            ibp.ibp_decompress(meta, comp.stream, comp.offsets, v.size, S, err=err)
            torch.cuda.synchronize()
            assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
        # the comparison codec's look-back, on a BF16 tensor of several blocks
        bf = rng.integers(0, 1 << 16, size=1_000_000, dtype=np.uint64).astype(np.uint16)
        xb = torch.from_numpy(bf.view(np.uint8).copy()).to(dev)
        table = ibp.ibp_zip_table_from_sigma(1e-3)
        for it in range(2):
            say(f"give-up path: exponent codec, wait limit 0, call {it}")
            err.zero_()
            z = ibp.ibp_zip_compress(table, xb, err=err)
            torch.cuda.synchronize()
            e = int(err.item())
            if e == 0:
                out = ibp.ibp_zip_decompress(z, err=err)
                torch.cuda.synchronize()
                assert torch.equal(out.view(torch.uint8), xb) and int(err.item()) == 0
                continue
            gave_up += 1
            assert e == ibp.IBP_DEVERR_TIMEOUT, e
            assert (z.eoff.cpu().numpy() == -1).any()
            err.zero_()
            ibp.ibp_zip_decompress(z, err=err)
            torch.cuda.synchronize()
            assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
    finally:
        ibp.ibp_set_wait_limit(0xFFFFFFFF)
    say(f"give-up path: {gave_up} of 6 calls gave up; default limit restored")
    err.zero_()
    comp = ibp.ibp_compress(meta, x, S, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off)
    assert np.array_equal(comp.stream[:nb].cpu().numpy(), ref_stream)


@pytest.mark.parametrize("tiles", [1, 15, 16, 17, 31, 32, 33, 255, 256, 257])
def test_lookback_status_layout_tile_counts(ibp, tiles):
    """Tile counts on both sides of the status layout's line counts (16 status words
    to a line over a power-of-two number of lines: a new line count from 16 * 2^k + 1
    tiles on), for the one-Mask compressor (8192-chunk tiles at W = 64), the
    position-metadata compressor (4096-chunk tiles) and the BF16 exponent codec
    (workgroups of 16,384 elements), each against the oracle; every input ends in a
    ragged last tile."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7000 + tiles)
    W, S = 64, 256
    mask, bitval = 0x7C007C007C007C00, 0x3800380038003800
    v = _data(rng, tiles * 8192 - 100, W, mask, bitval, 0.9)
    _run_case(ibp, dev, v, W, S, mask, bitval, f"{tiles} tiles")
    # position metadata: 4096-chunk tiles
    n = tiles * 4096 - 37
    masks = rng.integers(0, 1 << 62, S, dtype=np.uint64) & np.uint64(0xFFFF0000FFFF0000)
    bitvals = rng.integers(0, 1 << 62, S, dtype=np.uint64) & masks
    vp = rng.integers(0, 1 << 62, n, dtype=np.uint64)
    pos = np.arange(n) % S
    keep = rng.random(n) < 0.8
    vp[keep] = (vp[keep] & ~masks[pos[keep]]) | bitvals[pos[keep]]
    say(f"position tables: {tiles} tiles, n={n}")
    meta = ibp.PosMeta(W, S, torch.from_numpy(masks.view(np.int64)).to(dev),
                       torch.from_numpy(bitvals.view(np.int64)).to(dev))
    x = torch.from_numpy(vp.view(np.uint8).copy()).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ref_stream, ref_off = oracle.encode_pos(vp, W, masks, bitvals, S)
    comp = ibp.ibp_compress_pos(meta, x, err=err)
    assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), "position tables: offsets"
    assert np.array_equal(comp.stream[: ref_stream.size].cpu().numpy(), ref_stream), "position tables: stream"
    # BF16 exponent codec: workgroups of four 4096-element blocks
    m = tiles * 16384 - 5
    u = (rng.standard_normal(m).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    say(f"BF16 exponent codec: {tiles} workgroups, n={m}")
    table = oracle.zip_table(1.0)
    z = ibp.ibp_zip_compress(bytes(table), torch.from_numpy(u.view(np.int16).copy()).to(dev), err=err)
    sm, codes, esc, eoff = oracle.zip_encode(u, table)
    assert np.array_equal(z.eoff.cpu().numpy().view(np.uint64), eoff), "BF16 codec: escape offsets"
    assert np.array_equal(z.esc[: esc.size].cpu().numpy(), esc), "BF16 codec: escapes"
    torch.cuda.synchronize()
    assert int(err.item()) == 0
