"""Randomised GPU parity: seeded random configurations (W, S, size, Mask, Bitval,
share of matching chunks, per-position tables, fixed-slot tables) compressed,
decompressed and gathered by the HIP path and compared with the oracle byte for
byte.

The fixed grids of the other parity tests cover the kernels' paths by design; these
cases draw their parameters at random (reproducibly: seed = case number) to reach
combinations the grids miss: S from 1 to 1024, sizes up to about 3e5 chunks with
ragged tails, Masks of every popcount and run structure, both compression tile
forms.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DT = {16: np.uint16, 32: np.uint32, 64: np.uint64}
ALL = 0xFFFFFFFFFFFFFFFF


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


def say(msg):
    print(msg, flush=True)


def _rand_words(rng, n, W):
    v = rng.integers(0, 1 << 32, size=n, dtype=np.uint64) | (rng.integers(0, 1 << 32, size=n, dtype=np.uint64) << 32)
    return v & np.uint64((1 << W) - 1 if W < 64 else ALL)


def _rand_mask(rng, W):
    """A Mask of random popcount and structure: random bits, runs, or a contiguous
    block at the top (an exponent or a zero high part)."""
    full = (1 << W) - 1
    kind = int(rng.integers(0, 4))
    if kind == 0:
        return int(_rand_words(rng, 1, W)[0]) & int(_rand_words(rng, 1, W)[0])  # ~W/4 bits
    if kind == 1:
        return int(_rand_words(rng, 1, W)[0])  # ~W/2 bits
    if kind == 2:  # a few runs
        m = 0
        for _ in range(int(rng.integers(1, 5))):
            a = int(rng.integers(0, W))
            ln = int(rng.integers(1, W - a + 1))
            m |= ((1 << ln) - 1) << a
        return m & full
    k = int(rng.integers(0, W + 1))  # the top k bits
    return (full >> (W - k)) << (W - k) if k else 0


def _case(seed):
    rng = np.random.default_rng(seed)
    W = int(rng.choice([16, 32, 64]))
    S = int(rng.choice([1, 2, 3, 7, 16, 32, 64, 96, 100, 128, 200, 256, 333, 512, 640, 1000, 1024]))
    n = int(rng.integers(1, 300_000))
    p = float(rng.choice([0.0, 0.3, 0.7, 0.95, 1.0]))
    return rng, W, S, n, p


def _data(rng, n, W, mask, bitval, p):
    v = _rand_words(rng, n, W)
    keep = rng.random(n) < p
    full = np.uint64((1 << W) - 1 if W < 64 else ALL)
    v[keep] = (v[keep] & (~np.uint64(mask) & full)) | np.uint64(bitval)
    return v.astype(DT[W])


@pytest.mark.parametrize("seed", range(256))
def test_random_single_mask(ibp, seed):
    rng, W, S, n, p = _case(seed)
    mask = _rand_mask(rng, W)
    bitval = int(_rand_words(rng, 1, W)[0]) & mask
    say(f"fuzz {seed}: W={W} S={S} n={n} p={p} mask={mask:#x}")
    dev = torch.device("cuda:0")
    v = _data(rng, n, W, mask, bitval, p)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    meta = ibp.make_meta(W, mask, bitval)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    nb = ref_stream.size
    for form, threshold in (("default tiles", ALL), ("two-half tiles", 0)):
        ibp.ibp_set_halves_min_chunks(threshold)
        try:
            comp = ibp.ibp_compress(meta, x, S, err=err)
        finally:
            ibp.ibp_set_halves_min_chunks(ALL)
        assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), f"{form}: offsets"
        got = comp.stream[:nb].cpu().numpy()
        if not np.array_equal(got, ref_stream):
            bad = int(np.nonzero(got != ref_stream)[0][0])
            raise AssertionError(f"{form}: stream differs first at byte {bad} of {nb}")
    out = ibp.ibp_decompress(meta, comp.stream, comp.offsets, n, S, err=err)
    assert torch.equal(out, x), "round trip"
    full = n // S
    if full:
        ids_np = rng.integers(0, full, int(rng.integers(1, 300))).astype(np.int64)
        rows = ibp.ibp_decompress_gather(meta, comp.stream, comp.offsets, S, torch.from_numpy(ids_np).to(dev),
                                         err=err, n_segments=full)
        want = v[: full * S].reshape(full, S)[ids_np]
        assert np.array_equal(rows.cpu().numpy().view(DT[W]).reshape(len(ids_np), S), want), "gather"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("seed", range(1000, 1128))
def test_random_position_tables(ibp, seed):
    rng, W, S, n, p = _case(seed)
    if seed % 3 == 0:
        # every position's invariant bits at the top (its free bits one run from bit 0)
        full = (1 << W) - 1
        ks = rng.integers(0, W + 1, S)
        masks = np.array([(full >> (W - int(k))) << (W - int(k)) if k else 0 for k in ks], np.uint64)
    else:
        masks = np.array([_rand_mask(rng, W) for _ in range(S)], np.uint64)
    bitvals = np.array([int(_rand_words(rng, 1, W)[0]) & int(m) for m in masks], np.uint64)
    say(f"fuzz pos {seed}: W={W} S={S} n={n} p={p}")
    dev = torch.device("cuda:0")
    v = _rand_words(rng, n, W)
    pos = np.arange(n) % S
    keep = rng.random(n) < p
    full_w = np.uint64((1 << W) - 1 if W < 64 else ALL)
    v[keep] = (v[keep] & (~masks[pos[keep]] & full_w)) | bitvals[pos[keep]]
    v = v.astype(DT[W])
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    meta = ibp.PosMeta(W, S, torch.from_numpy(masks.view(np.int64)).to(dev),
                       torch.from_numpy(bitvals.view(np.int64)).to(dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
    nb = ref_stream.size
    for form, threshold in (("default tiles", ALL), ("two-half tiles", 0)):
        ibp.ibp_set_halves_min_chunks(threshold)
        try:
            comp = ibp.ibp_compress_pos(meta, x, err=err)
        finally:
            ibp.ibp_set_halves_min_chunks(ALL)
        assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), f"{form}: offsets"
        got = comp.stream[:nb].cpu().numpy()
        if not np.array_equal(got, ref_stream):
            bad = int(np.nonzero(got != ref_stream)[0][0])
            raise AssertionError(f"{form}: stream differs first at byte {bad} of {nb}")
    out = ibp.ibp_decompress_pos(meta, comp.stream, comp.offsets, n, err=err)
    assert torch.equal(out, x), "round trip"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("seed", range(2000, 2064))
def test_random_slots(ibp, seed):
    """The fixed-slot layout: every row's flag and used slot bytes against the
    oracle, and a gather of random rows against the input (rows that are not whole
    16-byte blocks: refused with IBP_ERR_SIZE)."""
    rng, W, S, _, p = _case(seed)
    R = int(rng.integers(1, 3000))
    mask = _rand_mask(rng, W)
    bitval = int(_rand_words(rng, 1, W)[0]) & mask
    say(f"fuzz slots {seed}: W={W} S={S} rows={R} p={p} mask={mask:#x}")
    dev = torch.device("cuda:0")
    v = _data(rng, R * S, W, mask, bitval, p)
    x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
    meta = ibp.make_meta(W, mask, bitval)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    if (S * W // 8) % 16:
        # slot rows must be whole 16-byte blocks: refused on the host
        with pytest.raises(ibp.IBPError) as e:
            ibp.ibp_compress_slots(meta, x, S, err=err)
        assert e.value.status == ibp.IBP_ERR_SIZE
        return
    slots, flags = ibp.ibp_compress_slots(meta, x, S, err=err)
    ref_slots, ref_flags, used = oracle.encode_slots(v, W, mask, bitval, S)
    got_flags = flags.cpu().numpy().view(np.uint64)
    assert np.array_equal(got_flags[: ref_flags.size], ref_flags), "flags"
    got = slots.cpu().numpy()
    rb = S * W // 8
    for r in range(R):
        nb = (int(used[r]) + 7) // 8
        assert np.array_equal(got[r * rb: r * rb + nb], ref_slots[r * rb: r * rb + nb]), f"slot {r}"
    ids_np = rng.integers(0, R, int(rng.integers(1, 300))).astype(np.int64)
    out = ibp.ibp_decompress_gather_slots(meta, slots, flags, S, torch.from_numpy(ids_np).to(dev), err=err)
    assert np.array_equal(out.cpu().numpy().view(DT[W]).reshape(len(ids_np), S), v.reshape(R, S)[ids_np]), "gather"
    torch.cuda.synchronize()
    assert int(err.item()) == 0
