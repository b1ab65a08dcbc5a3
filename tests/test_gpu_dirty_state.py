"""Codec kernels started on dirty GPU state: right before each codec call a helper
kernel leaves every CU's LDS and its waves' vector registers holding a pattern
(all ones, or alternating bits), and the codec's results must still equal the
oracle's bit for bit.

A kernel that read an LDS word or a register lane it had not written in the same
workgroup would pick up the pattern in its first workgroups (after a clean kernel
it would see zeros and pass).  The inputs span several generations of
workgroups per CU (thousands of tiles), so every kernel's later workgroups also
start where an earlier workgroup of the same kernel ran."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dirty_state

pytestmark = pytest.mark.gpu

DT = {16: np.uint16, 32: np.uint32, 64: np.uint64}
ALL = 0xFFFFFFFFFFFFFFFF
PATTERNS = (0xFFFFFFFF, 0xA5A5A5A5)
BLOCKS = 512  # two 1024-thread workgroups per CU on 256 CUs


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


@pytest.fixture(scope="module")
def sink():
    dirty_state.load()
    return torch.empty(int(dirty_state.load().dirty_sink_bytes(BLOCKS)), dtype=torch.uint8, device="cuda:0")


def say(msg):
    print(msg, flush=True)


def test_helper_leaves_lds_dirty(sink):
    """The helper works: workgroups of a kernel launched right after it find its
    pattern in LDS they never wrote."""
    dev = torch.device("cuda:0")
    cs = torch.cuda.current_stream()
    for pattern in PATTERNS:
        count = torch.zeros(256, dtype=torch.int32, device=dev)
        dirty_state.dirty(sink, BLOCKS, pattern, cs)
        dirty_state.peek_lds(count, pattern, cs)
        c = count.cpu().numpy()
        say(f"dirty LDS words seen per workgroup (of 16384): median {int(np.median(c))}, min {int(c.min())}")
        assert (c > 0).mean() > 0.5, "the next kernel's LDS does not hold the pattern"


def _words(rng, n, W):
    v = rng.integers(0, 1 << 32, size=n, dtype=np.uint64) | (rng.integers(0, 1 << 32, size=n, dtype=np.uint64) << 32)
    return v & np.uint64((1 << W) - 1 if W < 64 else ALL)


def _matching(rng, n, W, masks, bitvals, S, p):
    """Random W-bit chunks; a share p of them take their position's Bitval under its Mask."""
    v = _words(rng, n, W)
    pos = np.arange(n) % S
    keep = rng.random(n) < p
    full = np.uint64((1 << W) - 1 if W < 64 else ALL)
    v[keep] = (v[keep] & (~masks[pos[keep]] & full)) | bitvals[pos[keep]]
    return v.astype(DT[W])


def _stream_equal(comp, ref_stream, ref_off, what):
    assert np.array_equal(comp.offsets.cpu().numpy().view(np.uint64), ref_off), f"{what}: offsets"
    nb = ref_stream.size
    got = comp.stream[:nb].cpu().numpy()
    if not np.array_equal(got, ref_stream):
        d = np.nonzero(got != ref_stream)[0]
        raise AssertionError(f"{what}: {d.size} stream bytes differ, first at {int(d[0])} of {nb}")


# (W, S, n, Mask, Bitval, share matching): one-image and two-half tiles, the
# 1024-thread tiles (64-bit chunks with more than 32 invariant bits), the W = 16
# pair form, S dividing 64 and S neither dividing nor divisible by 64
SINGLE = [
    (32, 128, (1 << 24) + 77, 0x78000000, 0x38000000, 0.95),
    (64, 256, (1 << 24) + 5, 0xFFFFFFFFFF000000, 0, 0.97),
    (64, 256, (1 << 24) + 3, 0x7800000078000000, 0x3800000038000000, 0.9),
    (16, 1024, (1 << 25) + 9, 0x7C00, 0x3000, 0.97),
    (32, 32, (1 << 24) + 1, 0xC0000000, 0x40000000, 0.9),
    (64, 100, (1 << 23) + 11, 0xFFF0000000000000, 0x3FF0000000000000, 0.9),
]


@pytest.mark.parametrize("W,S,n,mask,bitval,p", SINGLE)
def test_single_mask_on_dirty_state(ibp, sink, W, S, n, mask, bitval, p):
    rng = np.random.default_rng(W * 1000 + S)
    v = _matching(rng, n, W, np.array([mask], np.uint64), np.array([bitval], np.uint64), 1, p)
    ref_stream, ref_off = oracle.encode(v, W, mask, bitval, S)
    full = n // S
    ids_np = rng.integers(0, full, 50_000).astype(np.int64)
    want = v[: full * S].reshape(full, S)[ids_np]
    slots_ok = (S * W // 8) % 16 == 0
    if slots_ok:
        ref_slots, ref_flags, used = oracle.encode_slots(v[: full * S], W, mask, bitval, S)
    for pattern in PATTERNS:
        say(f"dirty single: W={W} S={S} n={n} pattern={pattern:#x}")
        _single_mask_case(ibp, sink, W, S, n, mask, bitval, v, ref_stream, ref_off, ids_np, want,
                          (ref_slots, ref_flags, used) if slots_ok else None, pattern)


def _single_mask_case(ibp, sink, W, S, n, mask, bitval, v, ref_stream, ref_off, ids_np, want, ref_sl, pattern):
    dev = torch.device("cuda:0")
    cs = torch.cuda.current_stream()
    x = torch.from_numpy(v.view(np.uint8)).to(dev)
    meta = ibp.make_meta(W, mask, bitval)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for form, threshold in (("default tiles", ALL), ("two-half tiles", 0)):
        ibp.ibp_set_halves_min_chunks(threshold)
        try:
            dirty_state.dirty(sink, BLOCKS, pattern, cs)
            comp = ibp.ibp_compress(meta, x, S, err=err)
        finally:
            ibp.ibp_set_halves_min_chunks(ALL)
        _stream_equal(comp, ref_stream, ref_off, form)
    dirty_state.dirty(sink, BLOCKS, pattern, cs)
    out = ibp.ibp_decompress(meta, comp.stream, comp.offsets, n, S, err=err)
    assert torch.equal(out, x), "round trip"
    del out
    full = n // S
    ids = torch.from_numpy(ids_np).to(dev)
    dirty_state.dirty(sink, BLOCKS, pattern, cs)
    rows = ibp.ibp_decompress_gather(meta, comp.stream, comp.offsets, S, ids, err=err, n_segments=full)
    assert np.array_equal(rows.cpu().numpy().view(DT[W]).reshape(len(ids_np), S), want), "gather"
    if ref_sl is not None:
        ref_slots, ref_flags, used = ref_sl
        xs = x[: full * S * W // 8]
        dirty_state.dirty(sink, BLOCKS, pattern, cs)
        slots, flags = ibp.ibp_compress_slots(meta, xs, S, err=err)
        assert np.array_equal(flags.cpu().numpy().view(np.uint64)[: ref_flags.size], ref_flags), "slot flags"
        got = slots.cpu().numpy().reshape(full, S * W // 8)
        ref = ref_slots.reshape(full, S * W // 8)
        nb = (used.astype(np.int64) + 7) // 8
        cols = np.arange(S * W // 8)[None, :] < nb[:, None]
        assert np.array_equal(got[cols], ref[cols]), "slot bytes"
        dirty_state.dirty(sink, BLOCKS, pattern, cs)
        rows = ibp.ibp_decompress_gather_slots(meta, slots, flags, S, ids, err=err)
        assert np.array_equal(rows.cpu().numpy().view(DT[W]).reshape(len(ids_np), S), want), "slot gather"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


# position-dependent metadata: S a multiple of 64 (one-image and, at W = 64,
# two-half tiles), S dividing 64, S neither; random tables with top-bit and
# scattered Masks (the AND-only and the run-walking payload forms)
POS = [
    (32, 128, (1 << 24) + 77, "top"),
    (32, 128, (1 << 24) + 77, "scattered"),
    (64, 256, (1 << 24) + 5, "top"),
    (64, 256, (1 << 24) + 5, "scattered"),
    (64, 32, (1 << 23) + 3, "scattered"),
    (16, 256, (1 << 24) + 9, "scattered"),
    (32, 100, (1 << 23) + 13, "scattered"),
]


@pytest.mark.parametrize("W,S,n,kind", POS)
def test_position_metadata_on_dirty_state(ibp, sink, W, S, n, kind):
    rng = np.random.default_rng(W * 7000 + S)
    full_w = (1 << W) - 1
    if kind == "top":
        ks = rng.integers(0, W + 1, S)
        masks = np.array([(full_w >> (W - int(k))) << (W - int(k)) if k else 0 for k in ks], np.uint64)
    else:
        masks = _words(rng, S, W) & _words(rng, S, W) | (_words(rng, S, W) & np.uint64(full_w ^ (full_w >> 3)))
    bitvals = _words(rng, S, W) & masks
    v = _matching(rng, n, W, masks, bitvals, S, 0.9)
    ref_stream, ref_off = oracle.encode_pos(v, W, masks, bitvals, S)
    for pattern in PATTERNS:
        say(f"dirty pos: W={W} S={S} n={n} {kind} pattern={pattern:#x}")
        _position_case(ibp, sink, W, S, n, masks, bitvals, v, ref_stream, ref_off, pattern)


def _position_case(ibp, sink, W, S, n, masks, bitvals, v, ref_stream, ref_off, pattern):
    dev = torch.device("cuda:0")
    cs = torch.cuda.current_stream()
    x = torch.from_numpy(v.view(np.uint8)).to(dev)
    meta = ibp.PosMeta(W, S, torch.from_numpy(masks.view(np.int64)).to(dev),
                       torch.from_numpy(bitvals.view(np.int64)).to(dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for form, threshold in (("default tiles", ALL), ("two-half tiles", 0)):
        ibp.ibp_set_halves_min_chunks(threshold)
        try:
            dirty_state.dirty(sink, BLOCKS, pattern, cs)
            comp = ibp.ibp_compress_pos(meta, x, err=err)
        finally:
            ibp.ibp_set_halves_min_chunks(ALL)
        _stream_equal(comp, ref_stream, ref_off, form)
    dirty_state.dirty(sink, BLOCKS, pattern, cs)
    out = ibp.ibp_decompress_pos(meta, comp.stream, comp.offsets, n, err=err)
    assert torch.equal(out, x), "round trip"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_zip_codec_on_dirty_state(ibp, sink):
    """The BF16 exponent codec: sign-mantissa bytes, code planes, escapes and escape
    offsets against the oracle, and the round trip."""
    n = (1 << 24) + 333
    sigma = 1e-3
    rng = np.random.default_rng(99)
    f = (rng.standard_normal(n) * sigma).astype(np.float32)
    f[rng.random(n) < 0.01] *= 1e3
    bf = (f.view(np.uint32) >> 16).astype(np.uint16)
    table = oracle.zip_table(sigma)
    sm, codes, esc, eoff = oracle.zip_encode(bf, table)
    dev = torch.device("cuda:0")
    cs = torch.cuda.current_stream()
    x = torch.from_numpy(bf.view(np.int16)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for pattern in PATTERNS:
        say(f"dirty zip: n={n} pattern={pattern:#x}")
        dirty_state.dirty(sink, BLOCKS, pattern, cs)
        z = ibp.ibp_zip_compress(bytes(table), x, err=err)
        assert np.array_equal(z.sm[:n].cpu().numpy(), sm), "sign-mantissa bytes"
        assert np.array_equal(z.codes.cpu().numpy()[: codes.size], codes), "code planes"
        assert np.array_equal(z.eoff.cpu().numpy().view(np.uint64), eoff), "escape offsets"
        assert np.array_equal(z.esc.cpu().numpy()[: esc.size], esc), "escapes"
        dirty_state.dirty(sink, BLOCKS, pattern, cs)
        out = ibp.ibp_zip_decompress(z, err=err)
        assert torch.equal(out, x), "round trip"
    torch.cuda.synchronize()
    assert int(err.item()) == 0
