"""bit_packing_amd -- Python binding of the MI355X Invariant Bit Packing codec.

Argument marshalling only: every step of the codec runs in the HIP kernels of
``libibp.so`` (built from ``csrc/`` for gfx950, C ABI in ``include/ibp.h``).
torch supplies device memory, pinned host memory and streams.  The functions
have the names of the C entry points:

* ``ibp_build_metadata`` -- Mask/Bitval from a sample batch (IBP page,
  "Algoritmo Core", step 1);
* ``ibp_compress`` -- fused size / look-back / pack compression (step 2);
* ``ibp_decompress`` -- device-resident decompression (step 3);
* ``ibp_decompress_gather`` -- rows decoded straight from pinned host memory
  over PCIe ("Integrazione del Sistema", PCIe transfer compression);
* ``ibp_compress_slots`` / ``ibp_decompress_gather_slots`` -- the fixed-slot
  (in-place) layout of the PCIe transfer mode: each row keeps a slot of its raw
  size, only the used part is read, a bit vector marks compressed rows;
* ``ibp_gather_raw`` -- the uncompressed zero-copy gather the codec is
  measured against.

There is no fallback: if ``libibp.so`` is missing or no GPU is present the calls
raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # imported first so that libibp.so binds to the HIP runtime torch loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
# IBP_SANITIZE_LIB=1 loads the build whose host code carries AddressSanitizer and
# UndefinedBehaviorSanitizer checks (build_library(sanitize=True); the process must
# preload the clang ASan runtime, see tests/sanitize.sh)
LIB_PATH = os.path.join(_HERE, "libibp_san.so" if os.environ.get("IBP_SANITIZE_LIB") == "1" else "libibp.so")

IBP_OK, IBP_ERR_INVALID_ARG, IBP_ERR_SIZE, IBP_ERR_CAPACITY, IBP_ERR_DEVICE = 0, 1, 2, 3, 4
IBP_DEVERR_CORRUPT, IBP_DEVERR_BAD_ID, IBP_DEVERR_TIMEOUT = 1, 2, 4
IBP_MAX_S = 1024
IBP_NOALLOC_SCRATCH_BYTES = 8 << 20  # device array behind ibp_compress_noalloc, per GPU

EXPORTS = (
    "ibp_status_str", "ibp_num_segments", "ibp_max_stream_bytes", "ibp_stream_bytes",
    "ibp_metadata_workspace_bytes", "ibp_compress_workspace_bytes", "ibp_build_metadata",
    "ibp_compress", "ibp_decompress", "ibp_decompress_gather", "ibp_gather_raw",
    "ibp_slot_flag_words", "ibp_compress_slots", "ibp_decompress_gather_slots",
    "ibp_metadata_pos_workspace_bytes", "ibp_build_metadata_pos", "ibp_compress_pos", "ibp_decompress_pos",
    "ibp_zip_table_from_sigma", "ibp_zip_blocks", "ibp_zip_codes_bytes", "ibp_zip_workspace_bytes",
    "ibp_zip_compress", "ibp_zip_decompress", "ibp_set_wait_limit", "ibp_set_halves_min_chunks",
    "ibp_compress_noalloc",
)


class ibp_meta_t(ctypes.Structure):
    """Mask and Bitval of a dataset; only the low W bits are used."""
    _fields_ = [("W", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("mask", ctypes.c_uint64), ("bitval", ctypes.c_uint64)]

    def __repr__(self):
        return f"ibp_meta_t(W={self.W}, mask={self.mask:#x}, bitval={self.bitval:#x})"


class ibp_pos_meta_t(ctypes.Structure):
    """Position-dependent metadata: Mask_i / Bitval_i (device arrays of S words) for
    chunk position i of every segment."""
    _fields_ = [("W", ctypes.c_uint32), ("S", ctypes.c_uint32),
                ("mask", ctypes.c_void_p), ("bitval", ctypes.c_void_p)]


@dataclass
class PosMeta:
    """ibp_pos_meta_t plus the device tensors that hold its tables (kept alive here)."""
    W: int
    S: int
    mask: torch.Tensor    # int64[S], device
    bitval: torch.Tensor  # int64[S], device

    def struct(self) -> ibp_pos_meta_t:
        return ibp_pos_meta_t(self.W, self.S, _ptr(self.mask), _ptr(self.bitval))


def make_meta(W: int, mask: int, bitval: int) -> ibp_meta_t:
    return ibp_meta_t(W, 0, mask, bitval)


class IBPError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_name(status)}")


_lib = None
_u64, _u32, _vp, _dbl, _int = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
_metap = ctypes.POINTER(ibp_meta_t)


def load_library() -> ctypes.CDLL:
    """Load libibp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(bit_packing_amd.build.build_library())")
        lib = ctypes.CDLL(LIB_PATH)
        lib.ibp_status_str.argtypes = [_int]
        lib.ibp_status_str.restype = ctypes.c_char_p
        lib.ibp_num_segments.argtypes = [_u64, _u32]
        lib.ibp_max_stream_bytes.argtypes = [_u64, _u32]
        lib.ibp_stream_bytes.argtypes = [_u64]
        lib.ibp_metadata_workspace_bytes.argtypes = [_u64, _u32]
        lib.ibp_compress_workspace_bytes.argtypes = [_u64, _u32]
        for f in ("ibp_num_segments", "ibp_max_stream_bytes", "ibp_stream_bytes",
                  "ibp_metadata_workspace_bytes", "ibp_compress_workspace_bytes"):
            getattr(lib, f).restype = _u64
        lib.ibp_build_metadata.argtypes = [_vp, _u64, _u32, _dbl, _metap, _vp, _vp, _u64, _vp]
        lib.ibp_compress.argtypes = [_metap, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _u64, _vp, _vp]
        lib.ibp_decompress.argtypes = [_metap, _vp, _u64, _vp, _u64, _u32, _vp, _vp, _vp]
        lib.ibp_decompress_gather.argtypes = [_metap, _vp, _u64, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_gather_raw.argtypes = [_vp, _u64, _u64, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_slot_flag_words.argtypes = [_u64]
        lib.ibp_slot_flag_words.restype = _u64
        lib.ibp_compress_slots.argtypes = [_metap, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_decompress_gather_slots.argtypes = [_metap, _vp, _u64, _u64, _u32, _vp, _vp, _u64, _vp, _vp, _vp]
        _posp = ctypes.POINTER(ibp_pos_meta_t)
        lib.ibp_metadata_pos_workspace_bytes.argtypes = [_u32, _u32]
        lib.ibp_metadata_pos_workspace_bytes.restype = _u64
        lib.ibp_build_metadata_pos.argtypes = [_vp, _u64, _u32, _u32, _dbl, _vp, _vp, _vp, _vp, _u64, _vp]
        lib.ibp_compress_pos.argtypes = [_posp, _vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp, _vp]
        lib.ibp_decompress_pos.argtypes = [_posp, _vp, _u64, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_zip_table_from_sigma.argtypes = [_dbl, _vp]
        for f in ("ibp_zip_blocks", "ibp_zip_codes_bytes", "ibp_zip_workspace_bytes"):
            getattr(lib, f).argtypes = [_u64]
            getattr(lib, f).restype = _u64
        lib.ibp_zip_compress.argtypes = [_vp, _vp, _u64, _vp, _vp, _vp, _u64, _vp, _vp, _u64, _vp, _vp]
        lib.ibp_zip_decompress.argtypes = [_vp, _vp, _vp, _vp, _u64, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_compress_noalloc.argtypes = [_metap, _vp, _u64, _u32, _vp, _u64, _vp, _vp, _vp]
        lib.ibp_compress_noalloc.restype = _int
        lib.ibp_set_wait_limit.argtypes = [_u32]
        lib.ibp_set_wait_limit.restype = _u32
        lib.ibp_set_halves_min_chunks.argtypes = [_u64]
        lib.ibp_set_halves_min_chunks.restype = _u64
        for f in ("ibp_build_metadata", "ibp_compress", "ibp_decompress", "ibp_decompress_gather",
                  "ibp_gather_raw", "ibp_compress_slots", "ibp_decompress_gather_slots",
                  "ibp_build_metadata_pos", "ibp_compress_pos", "ibp_decompress_pos", "ibp_zip_table_from_sigma",
                  "ibp_zip_compress", "ibp_zip_decompress"):
            getattr(lib, f).restype = _int
        _lib = lib
    return _lib


def status_name(status: int) -> str:
    return load_library().ibp_status_str(status).decode()


def _check(rc: int, what: str) -> None:
    if rc != IBP_OK:
        raise IBPError(rc, what)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the codec must be contiguous")
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _device(*tensors) -> torch.device:
    for t in tensors:
        if t is not None and t.is_cuda:
            return t.device
    return torch.device("cuda", torch.cuda.current_device())


# ------------------------------------------------------------------ size queries

def ibp_num_segments(n_chunks: int, S: int) -> int:
    return int(load_library().ibp_num_segments(n_chunks, S))


def ibp_max_stream_bytes(n_chunks: int, W: int) -> int:
    return int(load_library().ibp_max_stream_bytes(n_chunks, W))


def ibp_stream_bytes(total_bits: int) -> int:
    return int(load_library().ibp_stream_bytes(total_bits))


def ibp_metadata_workspace_bytes(n_sample_chunks: int, W: int) -> int:
    return int(load_library().ibp_metadata_workspace_bytes(n_sample_chunks, W))


def ibp_compress_workspace_bytes(n_chunks: int, S: int) -> int:
    return int(load_library().ibp_compress_workspace_bytes(n_chunks, S))


def ibp_set_wait_limit(polls: int) -> int:
    """Tests of the compressors' give-up path only: look-back polls of one
    unpublished predecessor before a tile gives up (0xFFFFFFFF = the default).
    Returns the former value."""
    return int(load_library().ibp_set_wait_limit(polls))


def ibp_set_halves_min_chunks(n_chunks: int) -> int:
    """Compression inputs of at least n_chunks chunks (one Mask, W = 32 or 64, S a
    power of two) take the two-half tiles, smaller ones 8192-chunk tiles; the output
    is the same.  0xFFFFFFFFFFFFFFFF = the default (2^23).  Returns the former value."""
    return int(load_library().ibp_set_halves_min_chunks(n_chunks))


# ------------------------------------------------------------------ codec

def ibp_build_metadata(samples: torch.Tensor, W: int, T: float, stream=None,
                       workspace: torch.Tensor | None = None) -> tuple[ibp_meta_t, list[int]]:
    """(meta, per-position one-counts) of a device sample batch of W-bit chunks."""
    n = _nbytes(samples) // (W // 8) if W in (16, 32, 64) else 0
    if workspace is None:
        workspace = torch.empty(max(ibp_metadata_workspace_bytes(n, W), 8), dtype=torch.uint8,
                                device=_device(samples))
    meta = ibp_meta_t()
    counts = (ctypes.c_uint64 * 64)()
    rc = load_library().ibp_build_metadata(_ptr(samples), n, W, T, ctypes.byref(meta), counts,
                                           _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "ibp_build_metadata")
    return meta, [int(c) for c in counts[:W]]


@dataclass
class Compressed:
    """A compressed tensor: stream bytes, nseg + 1 bit offsets and the format parameters."""
    stream: torch.Tensor    # uint8, capacity >= used bytes
    offsets: torch.Tensor   # int64 bit offsets, nseg + 1 entries
    n_chunks: int
    S: int
    meta: ibp_meta_t


def ibp_compress(meta: ibp_meta_t, x: torch.Tensor, S: int, stream=None, err: torch.Tensor | None = None,
                 out_stream: torch.Tensor | None = None, out_offsets: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> Compressed:
    """Compress the bytes of x (read as W-bit little-endian chunks) with segments of S chunks."""
    W = meta.W
    n_bytes = _nbytes(x)
    n = n_bytes // (W // 8) if W in (16, 32, 64) else 0
    dev = _device(x)
    if out_stream is None:
        out_stream = torch.empty(max(ibp_max_stream_bytes(n, W), 16), dtype=torch.uint8, device=dev)
    if out_offsets is None:
        out_offsets = torch.empty(ibp_num_segments(n, S) + 1, dtype=torch.int64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(ibp_compress_workspace_bytes(n, S), 8), dtype=torch.uint8, device=dev)
    rc = load_library().ibp_compress(ctypes.byref(meta), _ptr(x), n_bytes, S, _ptr(out_stream),
                                     _nbytes(out_stream), _ptr(out_offsets), _ptr(workspace),
                                     _nbytes(workspace), _ptr(err), _stream(stream))
    _check(rc, "ibp_compress")
    return Compressed(out_stream, out_offsets, n, S, meta)


def ibp_decompress(meta: ibp_meta_t, stream_buf: torch.Tensor, offsets: torch.Tensor, n_chunks: int, S: int,
                   out: torch.Tensor | None = None, err: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decompress n_chunks chunks; returns out (uint8 unless an output tensor is given)."""
    if out is None:
        out = torch.empty(n_chunks * (meta.W // 8), dtype=torch.uint8, device=_device(offsets, stream_buf))
    rc = load_library().ibp_decompress(ctypes.byref(meta), _ptr(stream_buf), _nbytes(stream_buf), _ptr(offsets),
                                       n_chunks, S, _ptr(out), _ptr(err), _stream(stream))
    _check(rc, "ibp_decompress")
    return out


def ibp_decompress_gather(meta: ibp_meta_t, stream_buf: torch.Tensor, offsets: torch.Tensor, S: int,
                          ids: torch.Tensor, out: torch.Tensor | None = None, err: torch.Tensor | None = None,
                          stream=None, n_segments: int | None = None) -> torch.Tensor:
    """Row j of out (S chunks) = segment ids[j]; stream_buf may be pinned host memory."""
    if n_segments is None:
        n_segments = offsets.numel() - 1
    if out is None:
        out = torch.empty(ids.numel() * S * (meta.W // 8), dtype=torch.uint8, device=_device(ids, offsets))
    rc = load_library().ibp_decompress_gather(ctypes.byref(meta), _ptr(stream_buf), _nbytes(stream_buf),
                                              _ptr(offsets), n_segments, S, _ptr(ids), ids.numel(), _ptr(out),
                                              _ptr(err), _stream(stream))
    _check(rc, "ibp_decompress_gather")
    return out


def ibp_gather_raw(src: torch.Tensor, row_bytes: int, ids: torch.Tensor, out: torch.Tensor | None = None,
                   err: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Uncompressed zero-copy gather: row j of out = row ids[j] of src (rows of row_bytes bytes)."""
    n_rows = _nbytes(src) // row_bytes
    if out is None:
        out = torch.empty(ids.numel() * row_bytes, dtype=torch.uint8, device=_device(ids))
    rc = load_library().ibp_gather_raw(_ptr(src), row_bytes, n_rows, _ptr(ids), ids.numel(), _ptr(out),
                                       _ptr(err), _stream(stream))
    _check(rc, "ibp_gather_raw")
    return out


# ------------------------------------------------------------------ fixed-slot layout

def ibp_slot_flag_words(n_rows: int) -> int:
    return int(load_library().ibp_slot_flag_words(n_rows))


def ibp_compress_slots(meta: ibp_meta_t, x: torch.Tensor, S: int, slots: torch.Tensor | None = None,
                       flags: torch.Tensor | None = None, err: torch.Tensor | None = None,
                       stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Compress the rows of x (S chunks each) into fixed slots of their raw size.
    ``slots`` may be pinned host memory (compression in place in CPU memory).
    Returns (slots, flags): flags is one bit per row in int64 words (1 = compressed)."""
    row_bytes = S * meta.W // 8
    n_rows = _nbytes(x) // row_bytes if row_bytes else 0
    dev = _device(x)
    if slots is None:
        slots = torch.empty(max(n_rows * row_bytes, 16), dtype=torch.uint8, device=dev)
    if flags is None:
        flags = torch.empty(max(ibp_slot_flag_words(n_rows), 1), dtype=torch.int64, device=dev)
    rc = load_library().ibp_compress_slots(ctypes.byref(meta), _ptr(x), n_rows, S, _ptr(slots), _nbytes(slots),
                                           _ptr(flags), _ptr(err), _stream(stream))
    _check(rc, "ibp_compress_slots")
    return slots, flags


def ibp_decompress_gather_slots(meta: ibp_meta_t, slots: torch.Tensor, flags: torch.Tensor, S: int,
                                ids: torch.Tensor, n_rows: int | None = None, out: torch.Tensor | None = None,
                                err: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row j of out = row ids[j] of a slot table; slots may be pinned host memory."""
    row_bytes = S * meta.W // 8
    if n_rows is None:
        n_rows = _nbytes(slots) // row_bytes
    if out is None:
        out = torch.empty(ids.numel() * row_bytes, dtype=torch.uint8, device=_device(ids, flags))
    rc = load_library().ibp_decompress_gather_slots(ctypes.byref(meta), _ptr(slots), _nbytes(slots), n_rows, S,
                                                    _ptr(flags), _ptr(ids), ids.numel(), _ptr(out), _ptr(err),
                                                    _stream(stream))
    _check(rc, "ibp_decompress_gather_slots")
    return out


# ------------------------------------------------------------------ position-dependent metadata

def ibp_build_metadata_pos(samples: torch.Tensor, W: int, S: int, T: float, stream=None,
                           workspace: torch.Tensor | None = None, counts: bool = True) -> tuple[PosMeta, list | None]:
    """Mask_i / Bitval_i for the S chunk positions of a row, from device sample rows of S
    W-bit chunks.  Returns (PosMeta with device tables, counts[S][W] or None)."""
    n_rows = _nbytes(samples) // (S * W // 8) if W in (16, 32, 64) and S else 0
    dev = _device(samples)
    mask = torch.empty(max(S, 1), dtype=torch.int64, device=dev)
    bitval = torch.empty_like(mask)
    if workspace is None:
        workspace = torch.empty(max(int(load_library().ibp_metadata_pos_workspace_bytes(S, W)), 8),
                                dtype=torch.uint8, device=dev)
    host = (ctypes.c_uint64 * (S * W))() if counts else None
    rc = load_library().ibp_build_metadata_pos(_ptr(samples), n_rows, S, W, T, _ptr(mask), _ptr(bitval), host,
                                               _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, "ibp_build_metadata_pos")
    cl = [[host[i * W + b] for b in range(W)] for i in range(S)] if counts else None
    return PosMeta(W, S, mask, bitval), cl


def ibp_compress_pos(meta: PosMeta, x: torch.Tensor, stream=None, err: torch.Tensor | None = None,
                     out_stream: torch.Tensor | None = None, out_offsets: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> Compressed:
    """Compress the bytes of x with position-dependent metadata (segments of meta.S chunks)."""
    W, S = meta.W, meta.S
    n_bytes = _nbytes(x)
    n = n_bytes // (W // 8)
    dev = _device(x)
    if out_stream is None:
        out_stream = torch.empty(max(ibp_max_stream_bytes(n, W), 16), dtype=torch.uint8, device=dev)
    if out_offsets is None:
        out_offsets = torch.empty(ibp_num_segments(n, S) + 1, dtype=torch.int64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(ibp_compress_workspace_bytes(n, S), 8), dtype=torch.uint8, device=dev)
    st = meta.struct()
    rc = load_library().ibp_compress_pos(ctypes.byref(st), _ptr(x), n_bytes, _ptr(out_stream), _nbytes(out_stream),
                                         _ptr(out_offsets), _ptr(workspace), _nbytes(workspace), _ptr(err),
                                         _stream(stream))
    _check(rc, "ibp_compress_pos")
    return Compressed(out_stream, out_offsets, n, S, None)


def ibp_decompress_pos(meta: PosMeta, stream_buf: torch.Tensor, offsets: torch.Tensor, n_chunks: int,
                       out: torch.Tensor | None = None, err: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decompress n_chunks chunks encoded with position-dependent metadata."""
    if out is None:
        out = torch.empty(n_chunks * (meta.W // 8), dtype=torch.uint8, device=_device(offsets, stream_buf))
    st = meta.struct()
    rc = load_library().ibp_decompress_pos(ctypes.byref(st), _ptr(stream_buf), _nbytes(stream_buf), _ptr(offsets),
                                           n_chunks, _ptr(out), _ptr(err), _stream(stream))
    _check(rc, "ibp_decompress_pos")
    return out


# ------------------------------------------------------------------ comparison codec: BF16 exponent coding

@dataclass
class ZipCompressed:
    """BF16 exponent coding of n words: sign-mantissa bytes, code planes, escape
    exponents (capacity n; the first eoff[-1] are used) and per-block escape offsets."""
    sm: torch.Tensor
    codes: torch.Tensor
    esc: torch.Tensor
    eoff: torch.Tensor
    n: int
    table: bytes


def ibp_zip_table_from_sigma(sigma: float) -> bytes:
    t = (ctypes.c_uint8 * 7)()
    _check(load_library().ibp_zip_table_from_sigma(sigma, t), "ibp_zip_table_from_sigma")
    return bytes(t)


def _table_buf(table) -> ctypes.Array:
    t = bytes(table)
    if len(t) != 7:
        raise ValueError("a table is 7 exponents")
    return (ctypes.c_uint8 * 7)(*t)


def ibp_zip_compress(table, x: torch.Tensor, err: torch.Tensor | None = None, stream=None,
                     out: ZipCompressed | None = None, workspace: torch.Tensor | None = None) -> ZipCompressed:
    """Compress the BF16 words of x (any 2-byte dtype)."""
    lib = load_library()
    n = _nbytes(x) // 2
    dev = _device(x)
    if out is None:
        out = ZipCompressed(torch.empty(max(n, 16), dtype=torch.uint8, device=dev),
                            torch.empty(max(int(lib.ibp_zip_codes_bytes(n)), 16), dtype=torch.uint8, device=dev),
                            torch.empty(max(n, 16), dtype=torch.uint8, device=dev),
                            torch.empty(int(lib.ibp_zip_blocks(n)) + 1, dtype=torch.int64, device=dev), n, bytes(table))
    if workspace is None:
        workspace = torch.empty(max(int(lib.ibp_zip_workspace_bytes(n)), 8), dtype=torch.uint8, device=dev)
    rc = lib.ibp_zip_compress(_table_buf(table), _ptr(x), n, _ptr(out.sm), _ptr(out.codes), _ptr(out.esc),
                              _nbytes(out.esc), _ptr(out.eoff), _ptr(workspace), _nbytes(workspace), _ptr(err),
                              _stream(stream))
    _check(rc, "ibp_zip_compress")
    return out


def ibp_zip_decompress(z: ZipCompressed, out: torch.Tensor | None = None, err: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """BF16 words (as int16) of a ZipCompressed."""
    if out is None:
        out = torch.empty(max(z.n, 8), dtype=torch.int16, device=_device(z.sm))[: z.n]
    rc = load_library().ibp_zip_decompress(_table_buf(z.table), _ptr(z.sm), _ptr(z.codes), _ptr(z.esc),
                                           _nbytes(z.esc), _ptr(z.eoff), z.n, _ptr(out), _ptr(err), _stream(stream))
    _check(rc, "ibp_zip_decompress")
    return out
