"""Build and load tests/helpers/dirty_state.hip (a test helper that leaves the GPU's
LDS and vector registers at a pattern before a codec kernel runs)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dirty_state.hip")
LIB = os.path.join(HERE, "libdirty_state.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

_lib = None


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    subprocess.run([hipcc, *FLAGS, SRC, "-o", tmp], check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        lib.dirty_sink_bytes.argtypes = [ctypes.c_uint32]
        lib.dirty_sink_bytes.restype = ctypes.c_uint64
        lib.dirty_device_state.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        lib.dirty_device_state.restype = ctypes.c_int
        lib.dirty_peek_lds.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        lib.dirty_peek_lds.restype = ctypes.c_int
        _lib = lib
    return _lib


def dirty(sink, blocks: int, pattern: int, stream) -> None:
    """Queue the dirtying kernel on `stream` (a torch stream); sink: a device tensor of
    at least dirty_sink_bytes(blocks) bytes."""
    lib = load()
    assert sink.numel() * sink.element_size() >= lib.dirty_sink_bytes(blocks)
    rc = lib.dirty_device_state(ctypes.c_void_p(sink.data_ptr()), blocks, pattern & 0xFFFFFFFF,
                                ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"dirty_device_state: hip error {rc}")


def peek_lds(count, pattern: int, stream) -> None:
    """Queue a kernel of count.numel() workgroups that count the words of their unwritten
    LDS holding `pattern` (count: a zeroed int32 device tensor)."""
    rc = load().dirty_peek_lds(ctypes.c_void_p(count.data_ptr()), count.numel(), pattern & 0xFFFFFFFF,
                               ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"dirty_peek_lds: hip error {rc}")
