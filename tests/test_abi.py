"""The C ABI without a GPU: libibp.so loads, exports every entry point that
include/ibp.h declares, answers the size queries, and rejects bad arguments on
the host before any HIP call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ibp.h")


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    if not os.path.exists(bit_packing_amd.LIB_PATH):
        from bit_packing_amd.build import build_library
        build_library()
    bit_packing_amd.load_library()
    return bit_packing_amd


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"IBP_API\s+[\w\s\*]+?\b(ibp_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("ibp_build_metadata", "ibp_compress", "ibp_decompress", "ibp_decompress_gather"):
        assert s in syms


def test_every_declared_symbol_is_exported(ibp):
    lib = ibp.load_library()
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} declared in ibp.h but not exported"
    assert set(declared_symbols()) == set(ibp.EXPORTS)


def test_size_queries(ibp):
    assert ibp.ibp_num_segments(0, 256) == 0
    assert ibp.ibp_num_segments(257, 256) == 2
    assert ibp.ibp_num_segments(10, 0) == 0
    # worst case n * (W + 1) bits, in bytes, rounded up to 16
    assert ibp.ibp_max_stream_bytes(1000, 32) == 4128
    assert ibp.ibp_max_stream_bytes(1, 64) == 16
    assert ibp.ibp_stream_bytes(0) == 0
    assert ibp.ibp_stream_bytes(1) == 16
    assert ibp.ibp_stream_bytes(129) == 32
    # 8 bytes of control words, then for T compression tiles of 4096 chunks (whole
    # segments) the look-back status words, 16 to a line over the smallest power-of-two
    # number of lines that holds T, and T hand-over words
    assert ibp.ibp_compress_workspace_bytes(0, 256) == 8  # the control words only
    assert ibp.ibp_compress_workspace_bytes(4096, 256) == 8 + 8 * (16 + 1)
    assert ibp.ibp_compress_workspace_bytes(4097, 256) == 8 + 8 * (16 + 2)
    assert ibp.ibp_compress_workspace_bytes(4096, 1000) == 8 + 8 * (16 + 2)  # 4 segments of 1000 per tile
    assert ibp.ibp_compress_workspace_bytes(16 * 4096, 256) == 8 + 8 * (16 + 16)
    assert ibp.ibp_compress_workspace_bytes(17 * 4096, 256) == 8 + 8 * (32 + 17)
    assert ibp.ibp_compress_workspace_bytes(100 * 4096, 256) == 8 + 8 * (128 + 100)
    assert ibp.ibp_metadata_workspace_bytes(10, 64) == (64 + 66) * 8


def test_status_strings(ibp):
    assert ibp.status_name(0) == "IBP_OK"
    assert ibp.status_name(3) == "IBP_ERR_CAPACITY"
    assert ibp.status_name(99) == "IBP_ERR_UNKNOWN"


def _meta(ibp, W=32, mask=0xC0000000, bitval=0, reserved=0):
    return ibp.ibp_meta_t(W, reserved, mask, bitval)


FAKE = 0x10000  # never dereferenced: every call below fails its host checks first


def test_compress_argument_checks(ibp):
    lib = ibp.load_library()
    m = _meta(ibp)
    ok_ws = ibp.ibp_compress_workspace_bytes(1024, 256)
    cap = ibp.ibp_max_stream_bytes(1024, 32)
    call = lambda meta, n_bytes=4096, S=256, cap=cap, ws=ok_ws, inp=FAKE: lib.ibp_compress(
        ctypes.byref(meta), inp, n_bytes, S, FAKE, cap, FAKE, FAKE, ws, None, None)
    assert call(_meta(ibp, W=8, mask=0xC0)) == ibp.IBP_ERR_INVALID_ARG  # W not 16/32/64
    assert call(_meta(ibp, W=16)) == ibp.IBP_ERR_INVALID_ARG            # Mask wider than W = 16
    assert call(_meta(ibp, reserved=1)) == ibp.IBP_ERR_INVALID_ARG      # reserved must be 0
    assert call(_meta(ibp, bitval=0x1)) == ibp.IBP_ERR_INVALID_ARG      # Bitval outside Mask
    assert call(_meta(ibp, mask=1 << 40)) == ibp.IBP_ERR_INVALID_ARG    # Mask wider than W
    assert call(m, S=0) == ibp.IBP_ERR_INVALID_ARG
    assert call(m, S=ibp.IBP_MAX_S + 1) == ibp.IBP_ERR_INVALID_ARG
    assert call(m, n_bytes=4097) == ibp.IBP_ERR_SIZE                    # not whole chunks
    assert call(m, cap=cap - 16) == ibp.IBP_ERR_CAPACITY
    assert call(m, ws=ok_ws - 1) == ibp.IBP_ERR_CAPACITY
    assert call(m, inp=FAKE + 2) == ibp.IBP_ERR_INVALID_ARG             # misaligned input
    assert lib.ibp_compress(None, FAKE, 4096, 256, FAKE, cap, FAKE, FAKE, ok_ws, None, None) \
        == ibp.IBP_ERR_INVALID_ARG


def test_decompress_argument_checks(ibp):
    lib = ibp.load_library()
    m = _meta(ibp, W=64, mask=0xFF, bitval=0x12)
    assert lib.ibp_decompress(ctypes.byref(m), FAKE + 8, 4096, FAKE, 100, 256, FAKE, None, None) \
        == ibp.IBP_ERR_INVALID_ARG   # stream not 16-byte aligned
    assert lib.ibp_decompress(ctypes.byref(m), FAKE, 4096, FAKE, 100, 0, FAKE, None, None) \
        == ibp.IBP_ERR_INVALID_ARG   # S == 0
    assert lib.ibp_decompress(ctypes.byref(m), FAKE, 4096, None, 100, 256, FAKE, None, None) \
        == ibp.IBP_ERR_INVALID_ARG   # no offsets
    assert lib.ibp_decompress(ctypes.byref(m), FAKE, 4096, FAKE, 100, 256, FAKE + 4, None, None) \
        == ibp.IBP_ERR_INVALID_ARG   # output not aligned to W/8
    assert lib.ibp_decompress(ctypes.byref(m), FAKE, 4096, FAKE, 1 << 60, 256, FAKE, None, None) \
        == ibp.IBP_ERR_SIZE          # bit offsets would overflow
    assert lib.ibp_decompress_gather(ctypes.byref(m), FAKE, 4096, FAKE, 10, 32, None, 5, FAKE, None, None) \
        == ibp.IBP_ERR_INVALID_ARG   # ids missing
    assert lib.ibp_gather_raw(FAKE, 100, 10, FAKE, 5, FAKE, None, None) == ibp.IBP_ERR_SIZE


def test_metadata_argument_checks(ibp):
    lib = ibp.load_library()
    meta = ibp.ibp_meta_t()
    ws = ibp.ibp_metadata_workspace_bytes(100, 32)
    assert lib.ibp_build_metadata(FAKE, 100, 32, 0.5, ctypes.byref(meta), None, FAKE, ws, None) \
        == ibp.IBP_ERR_INVALID_ARG   # T must exceed 1/2
    assert lib.ibp_build_metadata(FAKE, 100, 32, 1.5, ctypes.byref(meta), None, FAKE, ws, None) \
        == ibp.IBP_ERR_INVALID_ARG
    assert lib.ibp_build_metadata(FAKE, 0, 32, 0.9, ctypes.byref(meta), None, FAKE, ws, None) \
        == ibp.IBP_ERR_INVALID_ARG   # empty sample
    assert lib.ibp_build_metadata(FAKE, 100, 8, 0.9, ctypes.byref(meta), None, FAKE, ws, None) \
        == ibp.IBP_ERR_INVALID_ARG   # W not 32/64
    assert lib.ibp_build_metadata(FAKE, 100, 32, 0.9, ctypes.byref(meta), None, FAKE, ws - 8, None) \
        == ibp.IBP_ERR_CAPACITY


def test_no_fallback_when_library_missing(ibp, monkeypatch):
    """The binding raises instead of computing anything itself."""
    monkeypatch.setattr(ibp, "_lib", None)
    monkeypatch.setattr(ibp, "LIB_PATH", "/nonexistent/libibp.so")
    with pytest.raises(RuntimeError):
        ibp.load_library()


def test_zip_table_matches_oracle(ibp):
    """The library's own sigma -> exponent table (host code) equals the oracle's."""
    import numpy as np

    import oracle
    for sigma in np.geomspace(1e-8, 1e5, 80):
        assert list(ibp.ibp_zip_table_from_sigma(float(sigma))) == oracle.zip_table(float(sigma)).tolist(), sigma
    lib = ibp.load_library()
    assert lib.ibp_zip_table_from_sigma(0.0, (ctypes.c_uint8 * 7)()) == ibp.IBP_ERR_INVALID_ARG
    assert ibp.load_library().ibp_zip_blocks(4097) == 2 and lib.ibp_zip_codes_bytes(4097) == 3072
    assert lib.ibp_zip_workspace_bytes(4096) == 8 + 8 * 16  # one workgroup's status line
    assert lib.ibp_zip_workspace_bytes(4096 * 4 * 17) == 8 + 8 * 32  # 17 workgroups of four blocks
    t = (ctypes.c_uint8 * 7)(1, 2, 3, 4, 5, 6, 6)  # repeated exponent
    assert lib.ibp_zip_compress(t, FAKE, 16, FAKE, FAKE, FAKE, 16, FAKE, FAKE, 64, None, None) == ibp.IBP_ERR_INVALID_ARG


def test_byte_counts_that_overflow_are_refused(ibp):
    """Products of counts that do not fit 64 bits are refused with IBP_ERR_SIZE on the
    host, before any pointer is resolved (so fake pointers are never looked at)."""
    lib = ibp.load_library()
    m = _meta(ibp)
    # gather: 8 (n_segments + 1) and n_segments * S would wrap
    for nseg in (1 << 61, (1 << 64) - 1, (1 << 55) // 128):
        assert lib.ibp_decompress_gather(ctypes.byref(m), FAKE, 4096, FAKE, nseg, 128, FAKE, 4, FAKE, None,
                                         None) == ibp.IBP_ERR_SIZE, nseg
    # raw gather: row_bytes * n_rows, row_bytes * n_ids and 8 n_ids would wrap
    assert lib.ibp_gather_raw(FAKE, 16, 1 << 61, FAKE, 4, FAKE, None, None) == ibp.IBP_ERR_SIZE
    assert lib.ibp_gather_raw(FAKE, 1 << 40, 1 << 30, FAKE, 4, FAKE, None, None) == ibp.IBP_ERR_SIZE
    assert lib.ibp_gather_raw(FAKE, 16, 4, FAKE, 1 << 61, FAKE, None, None) == ibp.IBP_ERR_SIZE
    assert lib.ibp_gather_raw(FAKE, 16, 0, FAKE, 4, FAKE, None, None) == ibp.IBP_ERR_SIZE  # no rows to gather from
    # slots: row and id counts are bounded before any product
    assert lib.ibp_decompress_gather_slots(ctypes.byref(m), FAKE, 1 << 62, 1 << 61, 128, FAKE, FAKE, 4, FAKE, None,
                                           None) == ibp.IBP_ERR_SIZE
    assert lib.ibp_compress_slots(ctypes.byref(m), FAKE, 1 << 61, 128, FAKE, 1 << 62, FAKE, None, None) \
        == ibp.IBP_ERR_SIZE


def test_wait_limit_setter(ibp):
    """The test-only look-back bound: set, read back, restore the default."""
    lib = ibp.load_library()
    first = ibp.ibp_set_wait_limit(5)
    assert ibp.ibp_set_wait_limit(0) == 5
    assert ibp.ibp_set_wait_limit(0xFFFFFFFF) == 0
    assert ibp.ibp_set_wait_limit(0xFFFFFFFF) == 1 << 20
    assert first == 1 << 20
    assert lib.ibp_set_wait_limit(0xFFFFFFFF) == 1 << 20


def test_halves_min_chunks_setter(ibp):
    """The compression tile-form threshold: set, read back, restore the default."""
    lib = ibp.load_library()
    first = ibp.ibp_set_halves_min_chunks(7)
    assert ibp.ibp_set_halves_min_chunks(0) == 7
    assert ibp.ibp_set_halves_min_chunks(0xFFFFFFFFFFFFFFFF) == 0
    assert ibp.ibp_set_halves_min_chunks(0xFFFFFFFFFFFFFFFF) == 1 << 23
    assert first == 1 << 23
    assert lib.ibp_set_halves_min_chunks(0xFFFFFFFFFFFFFFFF) == 1 << 23


def test_noalloc_limit_and_refusal(ibp):
    """The header's limit of the no-alloc compression equals the binding's, and an
    input whose workspace exceeds it is refused on the host (IBP_ERR_CAPACITY) before
    any pointer is looked at."""
    text = open(HEADER).read()
    m = re.search(r"#define IBP_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ibp.IBP_NOALLOC_SCRATCH_BYTES
    lib = ibp.load_library()
    meta = _meta(ibp, W=64, mask=0xFF00)
    n = 1
    while ibp.ibp_compress_workspace_bytes(n, 1) <= ibp.IBP_NOALLOC_SCRATCH_BYTES:
        n *= 2
    rc = lib.ibp_compress_noalloc(ctypes.byref(meta), FAKE, n * 8, 1, FAKE, ibp.ibp_max_stream_bytes(n, 64), FAKE,
                                  None, None)
    assert rc == ibp.IBP_ERR_CAPACITY
    assert lib.ibp_compress_noalloc(ctypes.byref(meta), FAKE, 4096, 0, FAKE, 1 << 20, FAKE, None, None) \
        == ibp.IBP_ERR_INVALID_ARG
    assert lib.ibp_compress_noalloc(ctypes.byref(meta), FAKE, 4095, 256, FAKE, 1 << 20, FAKE, None, None) \
        == ibp.IBP_ERR_SIZE
