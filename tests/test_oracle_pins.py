"""Pins of the CPU oracle against things other than itself.

* exhaustive brute force on tiny W and n against the bit-string spec
  (``spec_bits.py``), plus seeded random cases up to W = 64;
* closed forms: an all-invariant input reaches the minimum size (one bit per
  chunk), random bits with an empty Mask cost exactly one extra bit per chunk,
  the compressed size is the sum over chunks of 1 + (W - popcount(Mask)) or
  1 + W;
* x86 BMI2 PEXT/PDEP for the extract and deposit steps;
* numpy ``unpackbits`` column sums for the metadata counts;
* the closed-form metadata of a 24-bit id stream held in int64;
* error paths (bad arguments, corrupt offset tables).
"""
import ctypes
import itertools
import os
import random
import subprocess

import numpy as np
import pytest

import oracle
from spec_bits import spec_decode, spec_encode, spec_meta, int_to_bits


def _all_meta(W):
    """Every (Mask, Bitval) pair with Bitval inside Mask."""
    for mask in range(1 << W):
        sub = mask
        while True:
            yield mask, sub
            if sub == 0:
                break
            sub = (sub - 1) & mask


@pytest.mark.parametrize("W", [1, 2, 3])
def test_exhaustive_vs_spec(W):
    """Every input of n <= 3 chunks, every Mask/Bitval, every S: oracle == spec, round trip."""
    metas = list(_all_meta(W))
    for n in range(0, 4):
        for vals in itertools.product(range(1 << W), repeat=n):
            x = np.array(vals, np.uint64)
            for mask, bitval in metas:
                for S in range(1, max(n, 1) + 1):
                    stream, off = oracle.encode(x, W, mask, bitval, S)
                    ref_bytes, ref_off = spec_encode(list(vals), W, mask, bitval, S)
                    assert off.tolist() == ref_off
                    assert bytes(stream) == ref_bytes
                    back = oracle.decode(stream, off, n, W, mask, bitval, S)
                    assert back.tolist() == list(vals)


def test_exhaustive_injective_w2():
    """Distinct inputs never share a (stream, offsets) pair, for fixed metadata and S."""
    W = 2
    for mask, bitval in _all_meta(W):
        for n in range(1, 5):
            for S in range(1, n + 1):
                seen = {}
                for vals in itertools.product(range(1 << W), repeat=n):
                    stream, off = oracle.encode(np.array(vals, np.uint64), W, mask, bitval, S)
                    key = (bytes(stream), tuple(off.tolist()))
                    assert key not in seen, (vals, seen.get(key))
                    seen[key] = vals


def test_random_vs_spec():
    rng = random.Random(7)
    for _ in range(1500):
        W = rng.choice([1, 3, 5, 7, 8, 11, 16, 23, 32, 41, 63, 64])
        n = rng.randint(0, 40)
        S = rng.randint(1, 12)
        kind = rng.random()
        if kind < 0.15:
            mask = 0
        elif kind < 0.3:
            mask = (1 << W) - 1
        else:
            mask = rng.getrandbits(W)
        bitval = rng.getrandbits(W) & mask
        vals = []
        for _ in range(n):
            v = rng.getrandbits(W)
            if rng.random() < 0.7:  # make most chunks match
                v = (v & ~mask) | bitval
            vals.append(v)
        x = np.array(vals, np.uint64)
        stream, off = oracle.encode(x, W, mask, bitval, S)
        ref_bytes, ref_off = spec_encode(vals, W, mask, bitval, S)
        assert off.tolist() == ref_off
        assert bytes(stream) == ref_bytes
        assert spec_decode(ref_bytes, ref_off, n, W, mask, bitval, S) == vals
        assert oracle.decode(stream, off, n, W, mask, bitval, S).tolist() == vals


@pytest.mark.parametrize("W", [1, 2, 3])
def test_meta_exhaustive_vs_spec(W):
    """Every sample multiset of N <= 5 chunks and several thresholds T."""
    for N in range(1, 6):
        for combo in itertools.combinations_with_replacement(range(1 << W), N):
            x = np.array(combo, np.uint64)
            samples = [int_to_bits(v, W) for v in combo]
            for T in (0.51, 0.6, 0.75, 0.8, 1.0):
                mask, bitval, _ = oracle.build_meta(x, W, T)
                ms, bs = spec_meta(samples, T)
                assert (int_to_bits(mask, W), int_to_bits(bitval, W)) == (ms, bs), (combo, T)


def test_threshold_values():
    # k = ceil(T * N) with T taken in parts per million
    assert oracle.threshold(4096, 0.99) == 4056
    assert oracle.threshold(1_280_000, 0.95) == 1_216_000
    assert oracle.threshold(3_200_000, 0.98) == 3_136_000
    assert oracle.threshold(262_144, 0.97) == 254_280
    assert oracle.threshold(1_000_000, 0.999) == 999_000
    assert oracle.threshold(20, 0.95) == 19
    assert oracle.threshold(5, 1.0) == 5
    assert oracle.threshold(3, 0.51) == 2
    assert oracle.threshold(10, 0.5) == 0  # T must exceed 1/2
    assert oracle.threshold(10, 1.01) == 0


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("W,n,S", [(32, 1000, 256), (64, 77, 8), (8, 13, 5), (16, 9, 1)])
def test_all_invariant_minimum_size(W, n, S):
    """All-zero samples make every bit invariant; all-zero data then costs 1 bit per chunk."""
    dt = {8: np.uint8, 16: np.uint16, 32: np.uint32, 64: np.uint64}[W]
    mask, bitval, _ = oracle.build_meta(np.zeros(50, dt), W, 0.99)
    assert mask == (1 << W) - 1 and bitval == 0
    stream, off = oracle.encode(np.zeros(n, dt), W, mask, bitval, S)
    assert int(off[-1]) == n
    expected = [0xFF] * (n // 8) + ([(1 << (n % 8)) - 1] if n % 8 else [])
    assert stream.tolist() == expected
    assert off.tolist() == [min(k * S, n) for k in range((n + S - 1) // S + 1)]


@pytest.mark.parametrize("W", [32, 64])
def test_random_bits_one_extra_bit_per_chunk(W):
    """Uniform random words leave no invariant bit; each chunk then costs W + 1 bits and
    each segment is its S participation bits (all ones) followed by its chunks verbatim."""
    rng = np.random.default_rng(11)
    dt = np.uint32 if W == 32 else np.uint64
    sample = rng.integers(0, 2**W, size=20000, dtype=dt) if W == 32 else \
        rng.integers(0, 2**63, size=20000, dtype=np.uint64) * 2 + rng.integers(0, 2, size=20000, dtype=np.uint64)
    mask, bitval, _ = oracle.build_meta(sample, W, 0.95)
    assert mask == 0 and bitval == 0
    S, nseg = 8, 37
    x = sample[: S * nseg]
    stream, off = oracle.encode(x, W, mask, bitval, S)
    assert int(off[-1]) == S * nseg * (W + 1)
    raw = x.view(np.uint8).reshape(nseg, S * W // 8)
    expected = np.concatenate([np.concatenate([[0xFF], r]) for r in raw]).astype(np.uint8)
    assert np.array_equal(stream, expected)


@pytest.mark.parametrize("W,dt", [(32, np.float32), (64, np.float32), (64, np.uint16), (16, np.uint16)])
def test_size_formula(W, dt):
    """total bits == sum over chunks of 1 + (match ? W - popcount(Mask) : W)."""
    rng = np.random.default_rng(3)
    if dt == np.float32:
        x = (rng.standard_normal(40000) * 0.02).astype(np.float32)
    else:
        x = rng.integers(0x3800, 0x3C00, size=40000, dtype=np.uint16)
        x[::97] ^= 0x4000  # a few elements leave the common exponent range
    mask, bitval, _ = oracle.build_meta(x[:4096], W, 0.95)
    words = x.view({16: np.uint16, 32: np.uint32, 64: np.uint64}[W]).astype(np.uint64)
    matched = ((words ^ np.uint64(bitval)) & np.uint64(mask)) == 0
    pc = bin(mask).count("1")
    expected = int(np.where(matched, 1 + W - pc, 1 + W).sum())
    stream, off = oracle.encode(x, W, mask, bitval, 100)
    assert int(off[-1]) == expected
    assert stream.size == (expected + 7) // 8
    assert 0 < matched.mean() < 1  # both kinds of chunk occur


def test_last_byte_padding_zero():
    x = np.array([5, 1, 7], np.uint64)
    stream, off = oracle.encode(x, 3, 0b100, 0b100, 2)
    total = int(off[-1])
    assert total % 8 != 0
    assert stream[-1] >> (total % 8) == 0


# ---------------------------------------------------------------- BMI2

def _bmi2(tmp_path_factory):
    if "bmi2" not in open("/proc/cpuinfo").read():
        pytest.skip("host CPU has no BMI2")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "helpers", "bmi2_ref.c")
    so = str(tmp_path_factory.mktemp("bmi2") / "libbmi2.so")
    subprocess.check_call(["gcc", "-O1", "-mbmi2", "-shared", "-fPIC", "-o", so, src])
    lib = ctypes.CDLL(so)
    for f in (lib.ref_pext, lib.ref_pdep):
        f.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        f.restype = ctypes.c_uint64
    return lib


@pytest.mark.parametrize("W", [32, 64])
def test_extract_deposit_match_bmi2(W, tmp_path_factory):
    """A matching chunk's payload is PEXT(v, ~Mask); decoding is PDEP(payload, ~Mask) | Bitval."""
    lib = _bmi2(tmp_path_factory)
    rng = random.Random(5)
    full = (1 << W) - 1
    for _ in range(400):
        mask = rng.getrandbits(W)
        bitval = rng.getrandbits(W) & mask
        F = ~mask & full
        v = (rng.getrandbits(W) & F) | bitval
        stream, off = oracle.encode(np.array([v], np.uint64), W, mask, bitval, 1)
        word = int.from_bytes(bytes(stream), "little")
        assert word & 1 == 1
        assert word >> 1 == lib.ref_pext(v, F)
        x = rng.getrandbits(W - bin(mask).count("1")) if F else 0
        # a stream holding one matching chunk with payload x decodes to PDEP(x, F) | Bitval
        nbits = 1 + bin(F).count("1")
        s2 = np.frombuffer(((x << 1) | 1).to_bytes((nbits + 7) // 8, "little"), np.uint8)
        back = oracle.decode(s2, np.array([0, nbits], np.uint64), 1, W, mask, bitval, 1)
        assert int(back[0]) == lib.ref_pdep(x, F) | bitval


# ---------------------------------------------------------------- metadata counts

@pytest.mark.parametrize("W,dt", [(32, np.float32), (64, np.uint16), (16, np.uint16), (8, np.uint8)])
def test_counts_vs_unpackbits(W, dt):
    rng = np.random.default_rng(1)
    if dt == np.float32:
        x = rng.standard_normal(3000).astype(np.float32)
    else:
        x = rng.integers(0, np.iinfo(dt).max, size=3000, dtype=dt)
    counts = oracle.count_ones(x, W)
    bits = np.unpackbits(x.view(np.uint8).reshape(-1, W // 8), axis=1, bitorder="little")
    assert counts.tolist() == bits.sum(axis=0).tolist()


def test_int_ids_closed_form():
    """Ids below 2^24 in int64: the top 40 bits are invariant zeros, the low 24 are not."""
    rng = np.random.default_rng(2)
    sample = rng.integers(0, 1 << 24, size=100_000, dtype=np.int64)
    mask, bitval, _ = oracle.build_meta(sample, 64, 0.999)
    assert mask == 0xFFFFFFFFFF000000 and bitval == 0
    data = rng.integers(0, 1 << 24, size=5000, dtype=np.int64)
    big = rng.random(5000) < 0.05
    data[big] = rng.integers(0, 1 << 40, size=int(big.sum()), dtype=np.int64)
    small = data < (1 << 24)
    stream, off = oracle.encode(data, 64, mask, bitval, 256)
    assert int(off[-1]) == int(np.where(small, 25, 65).sum())
    assert np.array_equal(oracle.decode(stream, off, data.size, 64, mask, bitval, 256, np.int64), data)


# ---------------------------------------------------------------- gather, segments, errors

def test_gather_and_segment():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(32 * 50) * 0.05).astype(np.float32)
    mask, bitval, _ = oracle.build_meta(x, 64, 0.9)
    S = 16
    stream, off = oracle.encode(x, 64, mask, bitval, S)
    ids = np.array([3, 0, 49, 3, 17], np.int64)
    rows = oracle.decode_gather(stream, off, S, ids, 64, mask, bitval, np.float32).reshape(len(ids), -1)
    xr = x.reshape(-1, S * 2)
    assert np.array_equal(rows, xr[ids])
    for k in (0, 7, 49):
        seg, nbits = oracle.encode_segment(x, 64, mask, bitval, S, k)
        assert nbits == int(off[k + 1] - off[k])
        bits = np.unpackbits(stream, bitorder="little")[int(off[k]):int(off[k + 1])]
        assert np.array_equal(np.unpackbits(seg, bitorder="little")[:nbits], bits)


def test_error_paths():
    x = np.arange(10, dtype=np.uint32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.encode(x, 32, 0xF, 0x10, 4)  # Bitval outside Mask
    assert e.value.rc == oracle.EARG
    with pytest.raises(oracle.OracleError):
        oracle.encode(x, 32, 0, 0, 0)  # S == 0
    with pytest.raises(oracle.OracleError):
        oracle.build_meta(x, 32, 0.5)  # T must exceed 1/2
    with pytest.raises(oracle.OracleError):
        oracle.encode(np.array([8], np.uint64), 3, 0, 0, 1)  # value wider than W
    stream, off = oracle.encode(x, 32, 0xFFFFFF00, 0, 4)
    bad = off.copy()
    bad[1] += 1
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(stream, bad, 10, 32, 0xFFFFFF00, 0, 4)
    assert e.value.rc == oracle.ECORRUPT
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode_gather(stream, off, 4, np.array([3], np.int64), 32, 0xFFFFFF00, 0)
    assert e.value.rc == oracle.ESIZE


# ---------------------------------------------------------------- fixed-slot layout

@pytest.mark.parametrize("W,S", [(32, 128), (64, 32), (8, 5), (16, 3)])
def test_slots_layout(W, S):
    """Flags follow the size formula, compressed slots start with the row's segment bits,
    raw slots hold the row verbatim, and every row reads back."""
    rng = np.random.default_rng(W + S)
    R = 300
    dt = {8: np.uint8, 16: np.uint16, 32: np.uint32, 64: np.uint64}[W]
    full = (1 << W) - 1
    mask = (0x7C007C007C007C00 if W == 64 else 0x78000000 if W == 32 else 0xF0 if W == 8 else 0x7C00) & full
    bitval = mask & 0x3838383838383838
    rows = []
    for r in range(R):
        p_match = 0.95 if r % 3 else 0.02  # every third row almost all raw chunks
        v = rng.integers(0, 1 << min(W, 62), size=S, dtype=np.uint64).astype(dt) if W < 64 else \
            rng.integers(0, 1 << 62, size=S, dtype=np.uint64) * np.uint64(4) + rng.integers(0, 4, size=S, dtype=np.uint64)
        keep = rng.random(S) < p_match
        v[keep] = (v[keep] & dt(~mask & full)) | dt(bitval)
        rows.append(v)
    x = np.concatenate(rows).astype(dt)
    slots, flags, used = oracle.encode_slots(x, W, mask, bitval, S)
    words = x.astype(np.uint64).reshape(R, S)
    matched = ((words ^ np.uint64(bitval)) & np.uint64(mask)) == 0
    pc = bin(mask).count("1")
    seg_bits = S + np.where(matched, W - pc, W).sum(axis=1)
    want_flags = seg_bits < S * W
    got_flags = np.array([(int(flags[r // 64]) >> (r % 64)) & 1 for r in range(R)], bool)
    assert np.array_equal(got_flags, want_flags) and 0 < want_flags.mean() < 1
    rb = S * W // 8
    sl = slots.reshape(R, rb)
    for r in range(R):
        if want_flags[r]:
            seg, nbits = oracle.encode_segment(x, W, mask, bitval, S, r)
            assert int(used[r]) == nbits == seg_bits[r]
            assert np.array_equal(np.unpackbits(sl[r], bitorder="little")[:nbits],
                                  np.unpackbits(seg, bitorder="little")[:nbits])
        else:
            assert int(used[r]) == S * W
            assert np.array_equal(sl[r], x.view(np.uint8).reshape(R, rb)[r])
    ids = rng.integers(0, R, size=500).astype(np.int64)
    back = oracle.decode_slots_gather(slots, flags, S, ids, W, mask, bitval, dt).reshape(500, S)
    assert np.array_equal(back, x.reshape(R, S)[ids])


# ------------------------------------------------------------------ position-dependent metadata

from spec_bits import spec_encode_pos, spec_meta_pos  # noqa: E402


def _pairs(W):
    """Every (mask, bitval) with bitval inside mask, for width W."""
    return [(m, b) for m in range(1 << W) for b in range(1 << W) if b & ~m == 0]


@pytest.mark.parametrize("W,S,nmax", [(2, 2, 4), (1, 3, 5)])
def test_pos_exhaustive_vs_spec(W, S, nmax):
    """Every per-position metadata assignment and every input up to nmax chunks: the
    oracle's stream and offsets equal the bit-string specification's, and decode back."""
    import itertools
    pairs = _pairs(W)
    for combo in itertools.product(pairs, repeat=S):
        masks = [p[0] for p in combo]
        bitvals = [p[1] for p in combo]
        for n in range(nmax + 1):
            for vals in itertools.product(range(1 << W), repeat=n):
                x = np.array(vals, np.uint64)
                stream, off = oracle.encode_pos(x, W, masks, bitvals, S)
                ref, ref_off = spec_encode_pos(list(vals), W, masks, bitvals, S)
                assert off.tolist() == ref_off
                assert bytes(stream.tolist()) == ref
                assert oracle.decode_pos(stream, off, n, W, masks, bitvals, S).tolist() == list(vals)


def test_pos_random_vs_spec():
    rng = np.random.default_rng(71)
    for _ in range(150):
        W = int(rng.choice([3, 5, 8, 16, 31, 32, 33, 64]))
        S = int(rng.integers(1, 7))
        n = int(rng.integers(0, 40))
        full = (1 << W) - 1
        masks = [int(rng.integers(0, 1 << 62)) & full for _ in range(S)]
        bitvals = [int(rng.integers(0, 1 << 62)) & m for m in masks]
        vals = [int(rng.integers(0, 1 << 62)) & full for _ in range(n)]
        # make about half the chunks match their position's invariant bits
        vals = [(v & ~masks[i % S]) | bitvals[i % S] if rng.random() < 0.5 else v for i, v in enumerate(vals)]
        x = np.array(vals, np.uint64)
        stream, off = oracle.encode_pos(x, W, masks, bitvals, S)
        ref, ref_off = spec_encode_pos(vals, W, masks, bitvals, S)
        assert off.tolist() == ref_off and bytes(stream.tolist()) == ref
        assert oracle.decode_pos(stream, off, n, W, masks, bitvals, S).tolist() == vals


@pytest.mark.parametrize("W,S", [(8, 1), (8, 5), (32, 128), (64, 3)])
def test_pos_meta_is_per_column_meta(W, S):
    """Position i's Mask/Bitval/counts equal the single-Mask rule applied to the column
    of i-th chunks, and equal the bit-string specification on a small case."""
    rng = np.random.default_rng(W + S)
    dt = {8: np.uint8, 32: np.uint32, 64: np.uint64}[W]
    R = 501
    base = rng.integers(0, 1 << min(W, 62), size=(R, S), dtype=np.uint64)
    bias = rng.integers(0, 1 << min(W, 62), size=S, dtype=np.uint64)
    keep = rng.random((R, S)) < 0.93
    rows = np.where(keep, base & bias, base).astype(dt)
    for T in (0.51, 0.9, 0.95):
        masks, bitvals, c1 = oracle.build_meta_pos(rows.reshape(-1), W, S, T)
        for i in range(S):
            m, b, c = oracle.build_meta(np.ascontiguousarray(rows[:, i]), W, T)
            assert (int(masks[i]), int(bitvals[i])) == (m, b)
            assert c1[i].tolist() == c.tolist()
    if W == 8 and S <= 5:
        small = rows[:40]
        strs = [[int_to_bits(int(v), W) for v in row] for row in small]
        masks, bitvals, _ = oracle.build_meta_pos(small.reshape(-1), W, S, 0.9)
        ref = spec_meta_pos(strs, 0.9)
        for i in range(S):
            assert int_to_bits(int(masks[i]), W) == ref[i][0] and int_to_bits(int(bitvals[i]), W) == ref[i][1]


@pytest.mark.parametrize("W,S", [(32, 128), (64, 7), (16, 33)])
def test_pos_equal_masks_is_single_mask(W, S):
    """With the same Mask/Bitval at every position the variant is the single-Mask codec."""
    rng = np.random.default_rng(5 * W + S)
    full = (1 << W) - 1
    mask = int(rng.integers(0, 1 << 62)) & full
    bitval = int(rng.integers(0, 1 << 62)) & mask
    n = 50 * S + 3
    x = rng.integers(0, 1 << 62, size=n, dtype=np.uint64) & np.uint64(full)
    hit = rng.random(n) < 0.7
    x[hit] = (x[hit] & np.uint64(~mask & full)) | np.uint64(bitval)
    s1, o1 = oracle.encode(x, W, mask, bitval, S)
    s2, o2 = oracle.encode_pos(x, W, [mask] * S, [bitval] * S, S)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_pos_size_formula():
    """total bits = n + sum over chunks of (W - [match] * popcount(Mask_position)),
    computed here with numpy bit counts."""
    rng = np.random.default_rng(9)
    W, S, n = 32, 10, 12_345
    masks = rng.integers(0, 1 << 32, size=S, dtype=np.uint64)
    bitvals = rng.integers(0, 1 << 32, size=S, dtype=np.uint64) & masks
    x = rng.integers(0, 1 << 32, size=n, dtype=np.uint64)
    pos = np.arange(n) % S
    hit = rng.random(n) < 0.6
    x[hit] = (x[hit] & ~masks[pos[hit]] & np.uint64(0xFFFFFFFF)) | bitvals[pos[hit]]
    match = (x & masks[pos]) == bitvals[pos]
    pc = np.unpackbits(masks.astype(">u8").view(np.uint8)).reshape(S, 64).sum(1)
    expect = n + int((W - match * pc[pos]).sum())
    off = oracle.offsets_pos(x, W, masks, bitvals, S)
    assert int(off[-1]) == expect
    stream, off2 = oracle.encode_pos(x.astype(np.uint32), W, masks, bitvals, S)
    assert np.array_equal(off, off2)
    assert np.array_equal(oracle.decode_pos(stream, off, n, W, masks, bitvals, S), x)


# ------------------------------------------------------------------ ZipCCL exponent codec (comparison)

def _bf16_exponents_of_normal(rng, sigma, n):
    """Exponent field of N(0, sigma^2) samples as float32 (the BF16 exponent before rounding)."""
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return ((x.view(np.uint32) >> 23) & 0xFF).astype(np.int64)


@pytest.mark.parametrize("sigma", [1e-5, 1e-3, 0.02, 1.0, 37.0])
def test_zip_table_matches_sampled_exponents(sigma):
    """The sigma-derived table (no histogram) equals the 7 most frequent exponents of a
    large Gaussian sample: the same set, and the same order for the leading codes."""
    rng = np.random.default_rng(int(sigma * 1e6) % 2**32)
    counts = np.bincount(_bf16_exponents_of_normal(rng, sigma, 4_000_000), minlength=256)
    top = [int(e) for e in np.argsort(-counts, kind="stable")[:7]]
    t = [int(e) for e in oracle.zip_table(sigma)]
    assert set(t) == set(top)
    assert t[:4] == top[:4]


def test_zip_table_vs_scipy_cdf():
    """Masses from scipy's normal CDF at the BF16 exponent boundaries give the same ranking."""
    from scipy.stats import norm
    for sigma in np.geomspace(1e-7, 1e4, 60):
        e = np.arange(1, 255)
        lo, hi = np.ldexp(1.0, e - 127), np.ldexp(1.0, e - 126)
        mass = 2 * (norm.cdf(hi / sigma) - norm.cdf(lo / sigma))
        mass = np.concatenate([[2 * norm.cdf(np.ldexp(1.0, -126) / sigma) - 1], mass, [0.0]])
        order = sorted(range(256), key=lambda k: (-mass[k], k))[:7]
        assert oracle.zip_table(float(sigma)).tolist() == order, sigma


def _zip_spec(u, table):
    """Independent numpy statement of readings Z1-Z6 for one array of BF16 words."""
    u = u.astype(np.uint32)
    e = (u >> 7) & 0xFF
    sm = (((u >> 8) & 0x80) | (u & 0x7F)).astype(np.uint8)
    lut = np.zeros(256, np.uint32)
    for k, t in enumerate(table):
        lut[t] = k + 1
    c = lut[e]
    n = u.size
    nblk = (n + 4095) // 4096
    planes = np.zeros((nblk, 3, 4096), np.uint8)
    pad = np.zeros(nblk * 4096, np.uint32)
    pad[:n] = c
    for p in range(3):
        planes[:, p, :] = ((pad >> p) & 1).reshape(nblk, 4096)
    codes = np.packbits(planes.reshape(nblk, 3, 4096), axis=2, bitorder="little").reshape(-1)
    esc = e[c == 0].astype(np.uint8)
    per_blk = np.bincount(np.nonzero(c == 0)[0] // 4096, minlength=nblk)
    eoff = np.concatenate([[0], np.cumsum(per_blk)]).astype(np.uint64)
    return sm, codes, esc, eoff


def test_zip_all_bf16_words_vs_spec():
    """Every one of the 65,536 BF16 bit patterns, shuffled over 16 blocks plus a ragged
    tail, encodes as the numpy statement says and decodes back."""
    rng = np.random.default_rng(3)
    u = np.concatenate([rng.permutation(65536), rng.integers(0, 65536, 1234)]).astype(np.uint16)
    table = oracle.zip_table(1e-3)
    sm, codes, esc, eoff = oracle.zip_encode(u, table)
    rsm, rcodes, resc, reoff = _zip_spec(u, table)
    assert np.array_equal(sm, rsm) and np.array_equal(codes, rcodes)
    assert np.array_equal(esc, resc) and np.array_equal(eoff, reoff)
    assert np.array_equal(oracle.zip_decode(sm, codes, esc, eoff, u.size, table), u)


def test_zip_size_and_errors():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100_003) * 1e-3).astype(np.float32)
    u = (x.view(np.uint32) >> 16).astype(np.uint16)
    table = oracle.zip_table(1e-3)
    sm, codes, esc, eoff = oracle.zip_encode(u, table)
    nblk = (u.size + 4095) // 4096
    e = (u >> 7) & 0xFF
    assert esc.size == int((~np.isin(e, table)).sum())
    assert codes.size == nblk * 1536 and sm.size == u.size and eoff.size == nblk + 1
    assert esc.size < 0.05 * u.size  # the top 7 exponents cover > 95% of N(0, sigma) data
    with pytest.raises(oracle.OracleError):
        oracle.zip_encode(u, [1, 2, 3, 4, 5, 6, 6])  # a repeated exponent is not a table
    bad = eoff.copy()
    bad[5] += 1
    with pytest.raises(oracle.OracleError):
        oracle.zip_decode(sm, codes, esc, bad, u.size, table)
