"""CPU oracle of the Invariant Bit Packing codec -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``ibp_oracle.c``: a plain, slow, bit-at-a-time C
definition of the codec written from the IBP technical summary "Riduzione del
Collo di Bottiglia della Memoria GPU con la Compressione Lossless per il ML"
(gist.science, paper 2605.30728), section "Algoritmo Core", steps 1-3.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library (``bit_packing_amd``)
never imports it, and the two share no code.

Every function takes and returns numpy arrays.  Chunks are W-bit words; byte
inputs (W a multiple of 8) are read as little-endian W/8-byte words.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, hand-worked fixtures, exhaustive brute force against an
independent bit-string spec, BMI2 pext/pdep); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ibp_oracle.c")
# IBP_SANITIZE_ORACLE=1 selects the AddressSanitizer + UndefinedBehaviorSanitizer build
# (build(sanitize=True); the process must preload gcc's libasan, see tests/sanitize.sh)
_SANITIZED = os.environ.get("IBP_SANITIZE_ORACLE") == "1"
_LIB = os.path.join(_HERE, "libibp_oracle_san.so" if _SANITIZED else "libibp_oracle.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

OK, EARG, ESIZE, ECAP, ECORRUPT = 0, 1, 2, 3, 5


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"oracle {what} failed with code {rc}")
        self.rc = rc


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libibp_oracle.so`` (sanitize:
    ``oracle/libibp_oracle_san.so``, instrumented with ASan and UBSan)."""
    lib = os.path.join(_HERE, "libibp_oracle_san.so" if sanitize else "libibp_oracle.so")
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fPIC", "-shared", "-Wall",
                               "-Wextra", *(SAN_FLAGS if sanitize else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


_lib = None
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_vp = ctypes.c_void_p
_u64 = ctypes.c_uint64
_uint = ctypes.c_uint
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True, sanitize=_SANITIZED)
        lib = ctypes.CDLL(_LIB)
        lib.ibpo_threshold.argtypes = [_u64, ctypes.c_double]
        lib.ibpo_threshold.restype = _u64
        lib.ibpo_count_ones.argtypes = [_vp, _int, _u64, _uint, _vp]
        lib.ibpo_meta_from_counts.argtypes = [_vp, _u64, _uint, ctypes.c_double, _u64p, _u64p]
        lib.ibpo_build_meta.argtypes = [_vp, _int, _u64, _uint, ctypes.c_double, _u64p, _u64p, _vp]
        lib.ibpo_offsets.argtypes = [_vp, _int, _u64, _uint, _u64, _u64, _u64, _vp]
        lib.ibpo_encode.argtypes = [_vp, _int, _u64, _uint, _u64, _u64, _u64, _vp, _vp, _u64]
        lib.ibpo_encode_segment.argtypes = [_vp, _int, _u64, _uint, _u64, _u64, _u64, _u64, _vp,
                                            _u64, _u64p]
        lib.ibpo_decode.argtypes = [_vp, _u64, _vp, _u64, _uint, _u64, _u64, _u64, _vp, _int]
        lib.ibpo_decode_gather.argtypes = [_vp, _u64, _vp, _u64, _u64, _vp, _u64, _uint, _u64,
                                           _u64, _vp, _int]
        lib.ibpo_encode_slots.argtypes = [_vp, _u64, _uint, _u64, _u64, _u64, _vp, _vp]
        lib.ibpo_slot_bits.argtypes = [_vp, _u64, _uint, _u64, _u64, _vp]
        lib.ibpo_slot_bits.restype = _u64
        lib.ibpo_decode_slots_gather.argtypes = [_vp, _u64, _uint, _u64, _u64, _u64, _vp, _vp, _u64, _vp, _int]
        lib.ibpo_build_meta_pos.argtypes = [_vp, _int, _u64, _uint, _u64, ctypes.c_double, _vp, _vp, _vp]
        lib.ibpo_offsets_pos.argtypes = [_vp, _int, _u64, _uint, _vp, _vp, _u64, _vp]
        lib.ibpo_encode_pos.argtypes = [_vp, _int, _u64, _uint, _vp, _vp, _u64, _vp, _vp, _u64]
        lib.ibpo_decode_pos.argtypes = [_vp, _u64, _vp, _u64, _uint, _vp, _vp, _u64, _vp, _int]
        lib.ibpo_zip_table.argtypes = [ctypes.c_double, _vp]
        lib.ibpo_zip_encode.argtypes = [_vp, _u64, _vp, _vp, _vp, _vp, _vp, _u64p]
        lib.ibpo_zip_decode.argtypes = [_vp, _vp, _vp, _u64, _vp, _u64, _vp, _vp]
        for f in ("ibpo_zip_table", "ibpo_zip_encode", "ibpo_zip_decode"):
            getattr(lib, f).restype = _int
        for f in ("ibpo_count_ones", "ibpo_meta_from_counts", "ibpo_build_meta", "ibpo_offsets",
                  "ibpo_encode", "ibpo_encode_segment", "ibpo_decode", "ibpo_decode_gather",
                  "ibpo_encode_slots", "ibpo_decode_slots_gather", "ibpo_build_meta_pos",
                  "ibpo_offsets_pos", "ibpo_encode_pos", "ibpo_decode_pos"):
            getattr(lib, f).restype = _int
        _lib = lib
    return _lib


def lib() -> ctypes.CDLL:
    """The loaded oracle library (for callers that run its C functions from several
    threads at once; ctypes releases the GIL during each call)."""
    return _load()


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _src(x: np.ndarray, W: int):
    """(pointer, is_bytes, n_chunks, keepalive) for a chunk source.

    uint64 arrays are read as one chunk per element (any W); any other dtype is
    read as raw little-endian bytes and W must be a multiple of 8.
    """
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint64 and W != 64:
        return _ptr(x), 0, x.size, x
    b = x.view(np.uint8).reshape(-1)
    if W % 8:
        raise ValueError("byte input needs W to be a multiple of 8")
    if b.size % (W // 8):
        raise OracleError(ESIZE, "chunking")
    return _ptr(b), 1, b.size // (W // 8), b


def threshold(N: int, T: float) -> int:
    """k = ceil(round(T*1e6) * N / 1e6): majority count needed for an invariant bit."""
    return int(_load().ibpo_threshold(N, T))


def count_ones(samples: np.ndarray, W: int) -> np.ndarray:
    p, isb, N, keep = _src(samples, W)
    c1 = np.zeros(64, np.uint64)
    rc = _load().ibpo_count_ones(p, isb, N, W, _ptr(c1))
    if rc:
        raise OracleError(rc, "count_ones")
    return c1[:W].copy()


def meta_from_counts(c1: np.ndarray, N: int, W: int, T: float) -> tuple[int, int]:
    c = np.zeros(64, np.uint64)
    c[:W] = np.asarray(c1, np.uint64)[:W]
    m, bv = _u64(0), _u64(0)
    rc = _load().ibpo_meta_from_counts(_ptr(c), N, W, T, ctypes.byref(m), ctypes.byref(bv))
    if rc:
        raise OracleError(rc, "meta_from_counts")
    return int(m.value), int(bv.value)


def build_meta(samples: np.ndarray, W: int, T: float) -> tuple[int, int, np.ndarray]:
    """(Mask, Bitval, per-position one-counts) from a sample batch (step 1)."""
    p, isb, N, keep = _src(samples, W)
    m, bv = _u64(0), _u64(0)
    c1 = np.zeros(64, np.uint64)
    rc = _load().ibpo_build_meta(p, isb, N, W, T, ctypes.byref(m), ctypes.byref(bv), _ptr(c1))
    if rc:
        raise OracleError(rc, "build_meta")
    return int(m.value), int(bv.value), c1[:W].copy()


def offsets(x: np.ndarray, W: int, mask: int, bitval: int, S: int) -> np.ndarray:
    """Bit offset table off[0..nseg] of the compressed stream of x."""
    p, isb, n, keep = _src(x, W)
    nseg = (n + S - 1) // S if S else 0
    off = np.zeros(nseg + 1, np.uint64)
    rc = _load().ibpo_offsets(p, isb, n, W, mask, bitval, S, _ptr(off))
    if rc:
        raise OracleError(rc, "offsets")
    return off


def encode(x: np.ndarray, W: int, mask: int, bitval: int, S: int) -> tuple[np.ndarray, np.ndarray]:
    """(stream bytes, bit offsets) of x (step 2).  len(stream) == ceil(total/8)."""
    off = offsets(x, W, mask, bitval, S)
    total = int(off[-1])
    p, isb, n, keep = _src(x, W)
    stream = np.zeros(max((total + 7) // 8, 1), np.uint8)
    rc = _load().ibpo_encode(p, isb, n, W, mask, bitval, S, _ptr(off), _ptr(stream), stream.size)
    if rc:
        raise OracleError(rc, "encode")
    return stream[: (total + 7) // 8].copy(), off


def encode_segment(x: np.ndarray, W: int, mask: int, bitval: int, S: int, k: int) -> tuple[np.ndarray, int]:
    """(bytes, bit count) of segment k alone, written from bit 0."""
    p, isb, n, keep = _src(x, W)
    cap = (S * (W + 1) + 7) // 8 + 1
    buf = np.zeros(cap, np.uint8)
    bits = _u64(0)
    rc = _load().ibpo_encode_segment(p, isb, n, W, mask, bitval, S, k, _ptr(buf), cap, ctypes.byref(bits))
    if rc:
        raise OracleError(rc, "encode_segment")
    return buf[: (bits.value + 7) // 8].copy(), int(bits.value)


def decode(stream: np.ndarray, off: np.ndarray, n: int, W: int, mask: int, bitval: int, S: int,
           out_dtype=None) -> np.ndarray:
    """Decompress n chunks (step 3).  Returns uint64 values, or bytes viewed as out_dtype."""
    stream = np.ascontiguousarray(stream, np.uint8)
    off = np.ascontiguousarray(off, np.uint64)
    if out_dtype is None or W % 8:
        out = np.zeros(max(n, 1), np.uint64)
        isb = 0
    else:
        out = np.zeros(max(n * (W // 8), 1), np.uint8)
        isb = 1
    sp = _ptr(stream) if stream.size else None
    rc = _load().ibpo_decode(sp, stream.size, _ptr(off), n, W, mask, bitval, S, _ptr(out), isb)
    if rc:
        raise OracleError(rc, "decode")
    if isb:
        return out[: n * (W // 8)].view(out_dtype)
    return out[:n]


def decode_gather(stream: np.ndarray, off: np.ndarray, S: int, ids: np.ndarray, W: int, mask: int,
                  bitval: int, out_dtype=None) -> np.ndarray:
    """Rows ids[j] (S chunks each) of a stream of full segments; row j of the result."""
    stream = np.ascontiguousarray(stream, np.uint8)
    off = np.ascontiguousarray(off, np.uint64)
    ids = np.ascontiguousarray(ids, np.int64)
    nseg = off.size - 1
    m = ids.size
    if out_dtype is None or W % 8:
        out = np.zeros(max(m * S, 1), np.uint64)
        isb = 0
    else:
        out = np.zeros(max(m * S * (W // 8), 1), np.uint8)
        isb = 1
    rc = _load().ibpo_decode_gather(_ptr(stream) if stream.size else None, stream.size, _ptr(off), nseg, S,
                                    _ptr(ids), m, W, mask, bitval, _ptr(out), isb)
    if rc:
        raise OracleError(rc, "decode_gather")
    if isb:
        return out[: m * S * (W // 8)].view(out_dtype)
    return out[: m * S]


# ------------------------------------------------------------------ fixed-slot layout

def encode_slots(x: np.ndarray, W: int, mask: int, bitval: int, S: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(slots bytes, 64-bit flag words, used bits per slot) of the rows of x (S chunks each)
    in the fixed-slot layout: a row that compresses keeps its segment bits at the start
    of its slot (flag 1), any other row is stored raw (flag 0)."""
    p, isb, n, keep = _src(x, W)
    if not isb or n % S:
        raise ValueError("slots need byte input of whole rows")
    R = n // S
    slots = np.zeros(max(n * W // 8, 1), np.uint8)
    flags = np.zeros(max((R + 63) // 64, 1), np.uint64)
    rc = _load().ibpo_encode_slots(p, R, W, mask, bitval, S, _ptr(slots), _ptr(flags))
    if rc:
        raise OracleError(rc, "encode_slots")
    used = np.array([_load().ibpo_slot_bits(_ptr(slots), r, W, mask, S, _ptr(flags)) for r in range(R)], np.uint64)
    return slots[: n * W // 8], flags[: (R + 63) // 64], used


def decode_slots_gather(slots: np.ndarray, flags: np.ndarray, S: int, ids: np.ndarray, W: int, mask: int,
                        bitval: int, out_dtype=np.uint8) -> np.ndarray:
    """Rows ids[j] of a fixed-slot table, decoded."""
    slots = np.ascontiguousarray(slots, np.uint8)
    flags = np.ascontiguousarray(flags, np.uint64)
    ids = np.ascontiguousarray(ids, np.int64)
    R = slots.size // (S * W // 8)
    out = np.zeros(max(ids.size * S * W // 8, 1), np.uint8)
    rc = _load().ibpo_decode_slots_gather(_ptr(slots), R, W, mask, bitval, S, _ptr(flags), _ptr(ids), ids.size,
                                          _ptr(out), 1)
    if rc:
        raise OracleError(rc, "decode_slots_gather")
    return out[: ids.size * S * W // 8].view(out_dtype)


# ------------------------------------------------------------------ position-dependent metadata

def _pos_tables(mask, bitval, S: int):
    m = np.ascontiguousarray(np.asarray(mask, np.uint64).reshape(-1))
    b = np.ascontiguousarray(np.asarray(bitval, np.uint64).reshape(-1))
    if m.size != S or b.size != S:
        raise ValueError("one Mask and one Bitval per position")
    return m, b


def build_meta_pos(samples: np.ndarray, W: int, S: int, T: float) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(Mask_i, Bitval_i, one-counts [S, W]) from sample rows of S chunks: position i's
    metadata is the step-1 rule applied to the i-th chunk of every sample row."""
    p, isb, n, keep = _src(samples, W)
    if n % S or n == 0:
        raise ValueError("samples must be whole rows of S chunks")
    mask = np.zeros(S, np.uint64)
    bitval = np.zeros(S, np.uint64)
    c1 = np.zeros(S * W, np.uint64)
    rc = _load().ibpo_build_meta_pos(p, isb, n // S, W, S, T, _ptr(mask), _ptr(bitval), _ptr(c1))
    if rc:
        raise OracleError(rc, "build_meta_pos")
    return mask, bitval, c1.reshape(S, W)


def offsets_pos(x: np.ndarray, W: int, mask, bitval, S: int) -> np.ndarray:
    """Bit offset table of x when chunk position i of a segment uses Mask_i / Bitval_i."""
    m, b = _pos_tables(mask, bitval, S)
    p, isb, n, keep = _src(x, W)
    off = np.zeros((n + S - 1) // S + 1, np.uint64)
    rc = _load().ibpo_offsets_pos(p, isb, n, W, _ptr(m), _ptr(b), S, _ptr(off))
    if rc:
        raise OracleError(rc, "offsets_pos")
    return off


def encode_pos(x: np.ndarray, W: int, mask, bitval, S: int) -> tuple[np.ndarray, np.ndarray]:
    """(stream bytes, bit offsets) of x under position-dependent metadata."""
    m, b = _pos_tables(mask, bitval, S)
    off = offsets_pos(x, W, m, b, S)
    p, isb, n, keep = _src(x, W)
    stream = np.zeros(max((int(off[-1]) + 7) // 8, 1), np.uint8)
    rc = _load().ibpo_encode_pos(p, isb, n, W, _ptr(m), _ptr(b), S, _ptr(off), _ptr(stream), stream.size)
    if rc:
        raise OracleError(rc, "encode_pos")
    return stream[: (int(off[-1]) + 7) // 8], off


def decode_pos(stream: np.ndarray, off: np.ndarray, n: int, W: int, mask, bitval, S: int,
               out_dtype=None) -> np.ndarray:
    """Decompress n chunks encoded under position-dependent metadata."""
    m, b = _pos_tables(mask, bitval, S)
    stream = np.ascontiguousarray(stream, np.uint8)
    off = np.ascontiguousarray(off, np.uint64)
    if out_dtype is None or W % 8:
        out = np.zeros(max(n, 1), np.uint64)
        isb = 0
    else:
        out = np.zeros(max(n * (W // 8), 1), np.uint8)
        isb = 1
    rc = _load().ibpo_decode_pos(_ptr(stream) if stream.size else None, stream.size, _ptr(off), n, W, _ptr(m),
                                 _ptr(b), S, _ptr(out), isb)
    if rc:
        raise OracleError(rc, "decode_pos")
    if isb:
        return out[: n * (W // 8)].view(out_dtype)
    return out[:n]


# ------------------------------------------------------------------ ZipCCL exponent codec (comparison)

ZIP_BLOCK = 4096


def zip_table(sigma: float) -> np.ndarray:
    """The 7 BF16 exponents of largest mass under N(0, sigma^2), code 1..7 order."""
    t = np.zeros(7, np.uint8)
    rc = _load().ibpo_zip_table(sigma, _ptr(t))
    if rc:
        raise OracleError(rc, "zip_table")
    return t


def zip_encode(x: np.ndarray, table) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(sm bytes, code planes, escape exponents, escape offsets per block) of BF16 words x."""
    x = np.ascontiguousarray(np.asarray(x).view(np.uint16).reshape(-1))
    t = np.ascontiguousarray(np.asarray(table, np.uint8))
    n = x.size
    nblk = (n + ZIP_BLOCK - 1) // ZIP_BLOCK
    sm = np.zeros(max(n, 1), np.uint8)
    codes = np.zeros(max(nblk * 1536, 1), np.uint8)
    esc = np.zeros(max(n, 1), np.uint8)
    eoff = np.zeros(nblk + 1, np.uint64)
    ne = _u64(0)
    rc = _load().ibpo_zip_encode(_ptr(x) if n else None, n, _ptr(t), _ptr(sm), _ptr(codes), _ptr(esc), _ptr(eoff),
                                 ctypes.byref(ne))
    if rc:
        raise OracleError(rc, "zip_encode")
    return sm[:n], codes[: nblk * 1536], esc[: ne.value], eoff


def zip_decode(sm, codes, esc, eoff, n: int, table) -> np.ndarray:
    sm = np.ascontiguousarray(sm, np.uint8)
    codes = np.ascontiguousarray(codes, np.uint8)
    esc = np.ascontiguousarray(esc, np.uint8)
    eoff = np.ascontiguousarray(eoff, np.uint64)
    t = np.ascontiguousarray(np.asarray(table, np.uint8))
    out = np.zeros(max(n, 1), np.uint16)
    rc = _load().ibpo_zip_decode(_ptr(sm) if sm.size else None, _ptr(codes) if codes.size else None,
                                 _ptr(esc) if esc.size else None, esc.size, _ptr(eoff), n, _ptr(t), _ptr(out))
    if rc:
        raise OracleError(rc, "zip_decode")
    return out[:n]
