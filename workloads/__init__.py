"""Seeded synthetic workloads for the IBP codec (inputs only, no codec arithmetic).

The IBP page measures on real GNN, DLRM and LLM data it does not name ("Risultati"
section); these generators stand in for them with the shapes and value
distributions of five workloads:

=====  ==========================================  ====  =====  ====  =========================
name   data                                        W     T      S     metadata sample
=====  ==========================================  ====  =====  ====  =========================
tiny   262,144 fp32 ~ N(0, 0.02) (1 MiB)            32    0.99   256   first 4,096 values
gnn    1,000,000 x 128 fp32, max(N(0,1), +0)       32    0.95   128   10,000 distinct rows
dlrm   10,000,000 x 64 fp32 ~ U(-0.05, 0.05)       64    0.98   32    100,000 distinct rows
llm    2^30 bf16 ~ N(0,1e-3), 0.1% N(0,1) outliers 64    0.97   256   first 2^20 elements
ids    500,000,000 int64 ~ U[0,2^24), 5% U[0,2^40)  64    0.999  256   first 1,000,000 (before
                                                                      the 5% replacement)
sparse 1,000,000 x 128 fp32, 95% +0, rest |N(0,1)|   32    0.9    128   10,000 distinct rows
llm16  the llm tensor (same bytes), one bf16/chunk  16    0.97   1024  first 2^20 elements
mixed  2,000,000 rows x (32 uint32 ids ~ U[0,2^20), 64    0.98   32    100,000 distinct rows
       then 32 fp32 ~ N(0,1))
=====  ==========================================  ====  =====  ====  =========================

The first five are the measured configurations; "sparse" is the sparse-feature
regime of the IBP page's "Risultati" section (a GNN cache whose features are
mostly exact zeros); "llm16" codes the llm tensor with one bf16 element per
chunk (W = 16) instead of four; "mixed" is a feature table whose rows put
categorical ids before dense features, so which bits are invariant depends on
the chunk's position in the row (the case per-position metadata is for).  gnn, dlrm and sparse rows are one segment each (S = one row) and are read back by gathers:
65,536 uniform row ids per step (gnn) and 32,768 Zipf(1.05) row ids per step (dlrm).
``scale`` shrinks the row/element counts (same distributions) for CPU-sized tests.
All randomness comes from ``gen.c`` (counter-based SplitMix64), keyed by
seed = 1000 + workload number, so the same bytes come out on any machine and
thread count.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_SANITIZED = os.environ.get("IBP_SANITIZE_ORACLE") == "1"  # ASan + UBSan build (tests/sanitize.sh)
_LIB = os.path.join(_HERE, "libibpgen_san.so" if _SANITIZED else "libibpgen.so")


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile gen.c into libibpgen.so (sanitize: libibpgen_san.so, with ASan and
    UBSan and without OpenMP)."""
    lib = os.path.join(_HERE, "libibpgen_san.so" if sanitize else "libibpgen.so")
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp"
        flags = (["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
                  "-Wno-unknown-pragmas"]
                 if sanitize else ["-O2", "-fopenmp"])
        subprocess.check_call(["gcc", "-std=c11", *flags, "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(sanitize=_SANITIZED)
        L = ctypes.CDLL(_LIB)
        u64, vp, dbl, uint = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double, ctypes.c_uint
        L.gen_key.argtypes = [u64, u64]
        L.gen_key.restype = u64
        L.gen_u64.argtypes = [u64, u64]
        L.gen_u64.restype = u64
        L.gen_normal_f32.argtypes = [u64, u64, dbl, vp]
        L.gen_relu_normal_f32.argtypes = [u64, u64, vp]
        L.gen_uniform_f32.argtypes = [u64, u64, dbl, dbl, vp]
        L.gen_sparse_abs_normal_f32.argtypes = [u64, u64, dbl, vp]
        L.gen_bf16_grad.argtypes = [u64, u64, dbl, dbl, vp]
        L.gen_ids.argtypes = [u64, u64, uint, vp]
        L.gen_replace_ids.argtypes = [u64, u64, dbl, uint, vp]
        L.gen_sample_rows.argtypes = [u64, u64, u64, vp]
        L.gen_sample_rows.restype = ctypes.c_int
        L.gen_uniform_ids.argtypes = [u64, u64, u64, vp]
        L.gen_feature_rows.argtypes = [u64, u64, uint, uint, uint, vp]
        L.gen_zipf_ids.argtypes = [u64, u64, dbl, u64, vp]
        L.gen_zipf_ids.restype = ctypes.c_int
        L.gen_take_rows.argtypes = [vp, u64, vp, u64, vp]
        _lib = L
    return _lib


def key(seed: int, tag: int) -> int:
    return int(_load().gen_key(seed, tag))


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    description: str
    W: int
    T: float
    S: int
    dtype: str        # element dtype of the data
    row_elems: int    # elements per row (gather workloads), else 0
    gather: int       # ids per gather step (gather workloads), else 0
    sigma: float = 0.0  # standard deviation of the bulk of a Gaussian tensor (0: not Gaussian)

    @property
    def seed(self) -> int:
        return 1000 + self.number


WORKLOADS = {
    "tiny": Workload(1, "tiny", "262,144 fp32 ~ N(0, 0.02) (1 MiB gradient-like tensor)", 32, 0.99, 256,
                     "float32", 0, 0),
    "gnn": Workload(2, "gnn", "GNN feature cache: 1,000,000 nodes x 128 fp32, 50% zeros, rest |N(0,1)|", 32, 0.95,
                    128, "float32", 128, 65536),
    "dlrm": Workload(3, "dlrm", "DLRM embedding table: 10,000,000 rows x 64 fp32 ~ U(-0.05, 0.05)", 64, 0.98, 32,
                     "float32", 64, 32768),
    "llm": Workload(4, "llm", "LLM gradient buffer: 2^30 bf16 ~ N(0, 1e-3) with 0.1% N(0,1) outliers", 64, 0.97, 256,
                    "uint16", 0, 0, 1e-3),
    "ids": Workload(5, "ids", "Integer id stream: 500,000,000 int64 ~ U[0, 2^24), 5% U[0, 2^40)", 64, 0.999, 256,
                    "int64", 0, 0),
    "sparse": Workload(6, "sparse", "Sparse GNN feature cache: 1,000,000 nodes x 128 fp32, 95% zeros, rest |N(0,1)|",
                       32, 0.9, 128, "float32", 128, 65536),
    "llm16": Workload(7, "llm16", "LLM gradient buffer (the llm tensor) coded per element: 2^30 bf16, W=16", 16, 0.97,
                      1024, "uint16", 0, 0, 1e-3),
    "mixed": Workload(8, "mixed", "Feature rows: 2,000,000 x (32 uint32 ids ~ U[0, 2^20), then 32 fp32 ~ N(0,1))", 64,
                      0.98, 32, "uint32", 64, 0),
}

FULL_SIZE = {"tiny": 262_144, "gnn": 1_000_000, "dlrm": 10_000_000, "llm": 1 << 30, "ids": 500_000_000,
             "sparse": 1_000_000, "llm16": 1 << 30, "mixed": 2_000_000}
SAMPLE_SIZE = {"tiny": 4096, "gnn": 10_000, "dlrm": 100_000, "llm": 1 << 20, "ids": 1_000_000, "sparse": 10_000,
               "llm16": 1 << 20, "mixed": 100_000}


@dataclass
class Instance:
    """One generated workload: data (numpy, host), the contiguous metadata sample,
    and the format parameters."""
    w: Workload
    data: np.ndarray
    sample: np.ndarray
    sample_rows: np.ndarray | None  # gather workloads: which rows were sampled

    @property
    def n_chunks(self) -> int:
        return self.data.nbytes // (self.w.W // 8)

    @property
    def row_bytes(self) -> int:
        return self.w.row_elems * self.data.dtype.itemsize


def size_at(name: str, scale: float) -> int:
    """Row count (gather workloads) or element count at a scale."""
    n = int(FULL_SIZE[name] * scale)
    if name in ("llm", "llm16"):
        n -= n % 4  # whole 64-bit chunks of bf16 (llm16 codes the same tensor)
    return max(n, 1 if name in ("gnn", "dlrm", "sparse", "mixed") else 64)


def generate(name: str, scale: float = 1.0) -> Instance:
    """Generate workload `name` with its element/row count multiplied by scale."""
    w = WORKLOADS[name]
    L = _load()
    n = size_at(name, scale)
    k_data = key(w.seed, 1)
    if name == "tiny":
        data = np.empty(n, np.float32)
        L.gen_normal_f32(k_data, n, 0.02, data.ctypes.data)
        sample = data[: min(SAMPLE_SIZE[name], n)].copy()
        return Instance(w, data, sample, None)
    if name == "gnn":
        data = np.empty((n, w.row_elems), np.float32)
        L.gen_relu_normal_f32(k_data, data.size, data.ctypes.data)
    elif name == "dlrm":
        data = np.empty((n, w.row_elems), np.float32)
        L.gen_uniform_f32(k_data, data.size, -0.05, 0.05, data.ctypes.data)
    elif name == "sparse":
        data = np.empty((n, w.row_elems), np.float32)
        L.gen_sparse_abs_normal_f32(k_data, data.size, 0.05, data.ctypes.data)
    elif name == "mixed":
        data = np.empty((n, w.row_elems), np.uint32)
        L.gen_feature_rows(k_data, n, 32, 32, 20, data.ctypes.data)
    elif name in ("llm", "llm16"):
        data = np.empty(n, np.uint16)
        L.gen_bf16_grad(key(WORKLOADS["llm"].seed, 1), n, 1e-3, 1e-3, data.ctypes.data)
        sample = data[: min(SAMPLE_SIZE[name], n)].copy()
        return Instance(w, data, sample, None)
    elif name == "ids":
        data = np.empty(n, np.int64)
        L.gen_ids(k_data, n, 24, data.ctypes.data)
        sample = data[: min(SAMPLE_SIZE[name], n)].copy()  # taken before the replacement
        L.gen_replace_ids(key(w.seed, 2), n, 0.05, 40, data.ctypes.data)
        return Instance(w, data, sample, None)
    else:
        raise KeyError(name)
    # row workloads: distinct uniformly sampled rows, copied contiguously
    m = min(max(int(SAMPLE_SIZE[name] * scale), 1), n) if scale < 1 else SAMPLE_SIZE[name]
    rows = np.empty(m, np.int64)
    rc = L.gen_sample_rows(key(w.seed, 3), n, m, rows.ctypes.data)
    if rc:
        raise RuntimeError("row sampling failed")
    sample = np.empty((m, w.row_elems), data.dtype)
    L.gen_take_rows(data.ctypes.data, data.shape[1] * data.itemsize, rows.ctypes.data, m, sample.ctypes.data)
    return Instance(w, data, sample, rows)


def gather_ids(name: str, n_rows: int, steps: int, per_step: int | None = None) -> np.ndarray:
    """Row ids of `steps` gather steps, shape (steps, per_step): uniform for gnn and
    sparse, Zipf(1.05) over ranks with a seeded rank -> row permutation for dlrm."""
    w = WORKLOADS[name]
    per_step = per_step or w.gather
    L = _load()
    out = np.empty((steps, per_step), np.int64)
    if name in ("gnn", "sparse"):
        for s in range(steps):
            L.gen_uniform_ids(key(w.seed * 1_000_000 + s, 4), n_rows, per_step, out[s].ctypes.data)
    elif name == "dlrm":
        rc = L.gen_zipf_ids(key(w.seed, 5), n_rows, 1.05, steps * per_step, out.ctypes.data)
        if rc:
            raise MemoryError("zipf table allocation failed")
    else:
        raise KeyError(name)
    return out
