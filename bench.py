"""Benchmark of the IBP codec on one MI355X: the five measured workloads in one run,
one JSON line.

The workloads (seeded synthetic stand-ins for the IBP page's GNN, DLRM and LLM
data, section "Risultati"):

====  ======  =====================================================  ==========================
 no.  name    data                                                   what is measured
====  ======  =====================================================  ==========================
 1    tiny    262,144 fp32 ~ N(0, 0.02), 1 MiB                       device compress + decompress
 2    gnn     1,000,000 x 128 fp32, 50% zeros, rest |N(0,1)|         gathers of 65,536 uniform rows
                                                                     from pinned host memory
 3    dlrm    10,000,000 x 64 fp32 ~ U(-0.05, 0.05)                  gathers of 32,768 Zipf(1.05)
                                                                     rows from pinned host memory
 4    llm     2^30 bf16 ~ N(0, 1e-3), 0.1% N(0, 1) outliers          HBM -> HBM compress, decompress
 5    ids     500,000,000 int64 ~ U[0, 2^24), 5% U[0, 2^40)          HBM -> HBM compress, decompress
====  ======  =====================================================  ==========================

The headline (``value``, ``roofline``, ``cpu_baseline``, ``config``) is workload 5,
the largest: a step is one device-resident decompression of the 4 GB id stream;
W untimed steps, then exactly K steps replayed from one HIP graph and bracketed by
synchronisations.  Every workload's own figures (its step rate, the kernel's
roofline, counter traffic when the committed profile matches the kernel sources,
the oracle's 1-thread and N-thread rates, bit-exact checks) are under
``configs``; two variants of the page's other modes are under ``variants``
(the sparse feature cache, the W = 16 coding of the llm tensor).

Rows of workloads 2 and 3 are read zero-copy from pinned host memory over PCIe in
the page's fixed-slot layout (each row in a slot of its raw size, only the used
part read, a bit per row in GPU memory marking compressed rows), and beside it
from the packed stream located by its offset table; both are compared with the
uncompressed zero-copy gather of the same rows and with the PCIe ceilings measured
in the same run.  The HBM-resident gather (the cache-compression mode) is
reported separately.  For workloads 4 and 5 the whole tensor is also brought from
pinned host memory into HBM by one decoder launch reading the stream zero-copy,
beside the raw tensor's hipMemcpyAsync (``whole_tensor_pcie``).

Roofline: algorithmic bytes per launch of the step kernel over its mean launch time
(HIP events on the launching stream): HBM kernels against 8 TB/s, PCIe kernels
against the 64 GB/s of a PCIe 5.0 x16 link (and against the measured ceiling).

The CPU oracle (plain bit-at-a-time C) is timed on the host's cores on bounded
samples of the same work, on one thread and on N threads (N = the cores this
process may use, at most OMP_NUM_THREADS), for metadata, compression and
decompression; its outputs double as bit-exact checks of the GPU results on those
samples.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IBP decompress effective GB/s (HBM- and PCIe-sourced) + compression ratio"
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, AMD published
PCIE_PEAK_GBPS = 64.0      # PCIe 5.0 x16, one direction, published link rate
CONFIG_ORDER = ["tiny", "gnn", "dlrm", "llm", "ids"]
VARIANTS = ["sparse", "llm16", "mixed"]
KERNEL_SOURCES = [os.path.join(ROOT, "bit_packing_amd", "csrc", f) for f in
                  ("ibp_device.h", "ibp_decode_loops.h", "ibp_internal.h", "ibp_meta.hip", "ibp_encode.hip",
                   "ibp_decode.hip", "ibp_decode_pos.hip", "ibp_slots.hip", "ibp_zip.hip", "ibp_api.hip")]
T0 = time.perf_counter()


def log(msg: str) -> None:
    print(f"[bench {time.perf_counter() - T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: // comments, trailing blanks and empty lines
    do not count, so a comment edit leaves committed counter summaries valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def committed_counters(workload: str, kind: str) -> dict | None:
    """Fields of profiles/counters_<workload>_<kind>.txt (the step kernel's counter
    summary) when it was taken on the current kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}_{kind}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return fields


class Timer:
    """HIP events over a timed region of back-to-back launches on the launching
    (current) stream.  The launches are queued behind a short spin kernel, so the GPU
    runs them without waiting for the host: the span from the first launch's start
    event to the last one's end event, divided by the launch count, is the kernel's
    average duration (plus the dispatch gap between consecutive kernels).
    Returns (span in seconds, mean milliseconds per launch)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.spin_per_ms = None

    def _hold(self, ms):
        torch = self.torch
        if self.spin_per_ms is None:
            self.a.record()
            torch.cuda._sleep(1_000_000)
            self.b.record()
            torch.cuda.synchronize()
            self.spin_per_ms = 1_000_000 / max(self.a.elapsed_time(self.b), 1e-3)
        torch.cuda._sleep(int(self.spin_per_ms * ms))

    def run(self, fn, n):
        torch = self.torch
        torch.cuda.synchronize()
        self._hold(5.0 + 0.1 * n)
        self.a.record()
        for i in range(n):
            fn(i)
        self.b.record()
        torch.cuda.synchronize()
        span_ms = self.a.elapsed_time(self.b)
        return span_ms / 1e3, span_ms / n

    def best(self, fn, n, runs=3):
        """Per-launch milliseconds of the fastest of `runs` timed regions of n launches."""
        return min(self.run(fn, n)[1] for _ in range(runs))


def graph_wall(torch, fn, first, k):
    """Wall time of the k launches fn(first), ..., fn(first + k - 1) replayed from one
    HIP graph: the host's per-call cost (argument checks, ctypes) does not gate the GPU.
    One untimed replay first; the timed replay is bracketed by synchronisations."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(k):
            fn(first + i)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def roofline(bound, alg_bytes, kernel_ms, kernel, counters=None, extra=None):
    peak = HBM_PEAK_GBPS if bound == "hbm" else PCIE_PEAK_GBPS
    achieved = alg_bytes / kernel_ms / 1e6
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": "GB/s", "frac": achieved / peak,
         "traffic": None, "kernel": kernel, "kernel_ms": kernel_ms, "algorithmic_bytes_per_launch": alg_bytes}
    if counters:
        key = "hbm_bytes_per_launch" if bound == "hbm" else "host_read_bytes_per_launch"
        try:
            r["traffic"] = float(counters[key])
            r["traffic_source"] = counters.get("source", "")
            r["traffic_vs_algorithmic"] = r["traffic"] / alg_bytes
        except (KeyError, ValueError):
            pass
    if extra:
        r.update(extra)
    return r


# ---------------------------------------------------------------------------- GPU side

class Ctx:
    def __init__(self, args):
        import torch

        import bit_packing_amd as ibp

        ibp.load_library()
        self.torch, self.ibp, self.args = torch, ibp, args
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.timer = Timer(torch)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.pcie = None

    def pcie_ceilings(self):
        """PCIe bandwidth measured in this run: hipMemcpyAsync H2D of 256 MiB from pinned
        memory, and a zero-copy streaming read of the same buffer by a kernel."""
        if self.pcie is None:
            torch, ibp = self.torch, self.ibp
            probe = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
            probe_d = torch.empty_like(probe, device=self.dev)
            _, cp_ms = self.timer.run(lambda i: probe_d.copy_(probe, non_blocking=True), 5)
            seq = torch.arange((256 << 20) // 4096, dtype=torch.int64, device=self.dev)
            _, zc_ms = self.timer.run(lambda i: ibp.ibp_gather_raw(probe, 4096, seq, out=probe_d), 5)
            cp, zc = probe.numel() / cp_ms / 1e6, probe.numel() / zc_ms / 1e6
            self.pcie = {"measured_GBps": max(cp, zc), "memcpy_h2d_GBps": cp, "zero_copy_stream_GBps": zc,
                         "pinned_allocation": "torch pin_memory (hipHostMalloc, flags 0: hipHostMallocDefault)"}
            del probe, probe_d
        return self.pcie

    def device_copy(self):
        torch = self.torch
        a = torch.empty(256 << 20, dtype=torch.uint8, device=self.dev)
        b = torch.empty_like(a)
        _, ms = self.timer.run(lambda i: b.copy_(a), 10)
        return {"GBps": 2 * (256 << 20) / ms / 1e6, "fraction_of_peak": 2 * (256 << 20) / ms / 1e6 / HBM_PEAK_GBPS}


def run_workload(ctx: Ctx, name: str, headline: bool) -> dict:
    import numpy as np

    import workloads

    torch, ibp, timer, err, args = ctx.torch, ctx.ibp, ctx.timer, ctx.err, ctx.args
    dev = ctx.dev
    w = workloads.WORKLOADS[name]
    inst = workloads.generate(name, args.scale)
    W, T, S = w.W, w.T, w.S
    n_chunks = inst.n_chunks
    U = inst.data.nbytes
    gather = w.gather > 0
    log(f"{name}: generated {U / 1e9:.3f} GB")
    rec = {"workload": f"{name}: {w.description}", "number": w.number, "W": W, "T": T, "S": S,
           "bytes": U, "chunks": n_chunks, "elements": int(inst.data.size)}
    checks = {}

    x = torch.from_numpy(inst.data.reshape(-1).view(np.uint8)).to(dev)
    sample = torch.from_numpy(inst.sample.reshape(-1).view(np.uint8)).to(dev)

    # step 1: metadata (synchronous by definition: wall time)
    meta, counts = ibp.ibp_build_metadata(sample, W, T)
    t0 = time.perf_counter()
    for _ in range(5):
        meta, counts = ibp.ibp_build_metadata(sample, W, T)
    rec["metadata"] = {"ms": (time.perf_counter() - t0) / 5 * 1e3, "sample_chunks": int(inst.sample.nbytes * 8 // W),
                       "mask": hex(meta.mask), "bitval": hex(meta.bitval)}

    # step 2: compression, HBM -> HBM
    cap = ibp.ibp_max_stream_bytes(n_chunks, W)
    stream_d = torch.empty(cap, dtype=torch.uint8, device=dev)
    nseg = ibp.ibp_num_segments(n_chunks, S)
    off_d = torch.empty(nseg + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(ibp.ibp_compress_workspace_bytes(n_chunks, S), dtype=torch.uint8, device=dev)

    def compress(_i):
        ibp.ibp_compress(meta, x, S, err=err, out_stream=stream_d, out_offsets=off_d, workspace=ws)

    compress(0)
    reps = 10 if U > (64 << 20) else 20
    c_ms = timer.best(compress, reps)
    total_bits = int(off_d[-1].item())
    C = (total_bits + 7) // 8
    c_alg = U + C + 8 * (nseg + 1)
    rec["compress"] = {"kernel_ms": c_ms, "effective_GBps": U / c_ms / 1e6, "algorithmic_GBps": c_alg / c_ms / 1e6,
                       "hbm_fraction": c_alg / c_ms / 1e6 / HBM_PEAK_GBPS}
    rec["ratio"] = {"r_stream": U / C, "r_total": U / (C + 8 * (nseg + 1) + 24), "stream_bytes": C,
                    "input_bytes": U, "segments": nseg}
    stream_bytes = ibp.ibp_stream_bytes(total_bits)
    stream_v = stream_d[:stream_bytes]
    log(f"{name}: ratio {U / C:.4f}, compress {c_ms:.3f} ms")

    # step 3: device-resident decompression of the whole tensor
    out_full = torch.empty_like(x)

    def decompress(_i):
        ibp.ibp_decompress(meta, stream_v, off_d, n_chunks, S, out=out_full, err=err)

    decompress(0)
    d_alg = C + 8 * (nseg + 1) + U
    if headline:
        for i in range(args.warmup):
            decompress(i)
        eager_wall, d_ms = timer.run(decompress, args.steps)
        wall = graph_wall(torch, decompress, 0, args.steps)
        rec["timed_step"] = {"steps": args.steps, "warmup": args.warmup, "graph_wall_s": wall,
                             "graph_ms_per_step": wall / args.steps * 1e3,
                             "eager_queued_ms_per_step": eager_wall / args.steps * 1e3}
        rec["value"] = U * args.steps / wall / 1e9
        rec["ms_per_step"] = wall / args.steps * 1e3
    else:
        d_ms = timer.best(decompress, reps)
    rec["decompress_device"] = {"kernel_ms": d_ms, "effective_GBps": U / d_ms / 1e6,
                                "algorithmic_GBps": d_alg / d_ms / 1e6,
                                "hbm_fraction": d_alg / d_ms / 1e6 / HBM_PEAK_GBPS}
    torch.cuda.synchronize()
    checks["roundtrip_equal"] = bool(torch.equal(out_full, x))
    del out_full
    log(f"{name}: decompress {d_ms:.3f} ms ({d_alg / d_ms / 1e6 / HBM_PEAK_GBPS:.3f} of HBM peak)")

    if not gather:
        if not headline:
            rec["value"] = U / d_ms / 1e6
            rec["ms_per_step"] = d_ms
        rec["step"] = "device-resident decompression of the whole tensor (HBM -> HBM)"
        rec["roofline"] = roofline("hbm", d_alg, d_ms, "ibp_decompress (decode_kernel)",
                                   committed_counters(name, "decompress"))
        if name == "tiny":
            rec["roofline"]["note"] = ("about 2 MB per launch: launch- and cache-bound, reported but not a "
                                       "bandwidth case")
        rec["roofline_compress"] = roofline("hbm", c_alg, c_ms, "ibp_compress (encode_kernel)",
                                            committed_counters(name, "compress"))
    else:
        gather_section(ctx, name, inst, meta, x, stream_v, off_d, C, nseg, U, rec, checks, headline)

    if name in ("llm", "mixed"):
        position_metadata_variant(ctx, inst, x, sample, meta, S, rec, checks)
    if name == "llm":
        zipccl_variant(ctx, inst, x, rec, checks)
    if name in ("llm", "ids"):
        whole_tensor_transfer(ctx, meta, x, stream_v, off_d, n_chunks, S, C, nseg, U, rec, checks)
    if name == "gnn":
        zero_copy_compress(ctx, meta, inst, x, S, stream_d, off_d, ws, C, rec, checks)

    torch.cuda.synchronize()
    rec["device_error_word"] = int(err.item())
    if not args.no_cpu_baseline:
        log(f"{name}: oracle baseline")
        rec["cpu_baseline"] = cpu_baseline(inst, meta, stream_d, off_d, total_bits, counts, args.cpu_seconds,
                                           checks)
    rec["checks"] = checks
    del x, sample, stream_d, off_d, ws, stream_v
    torch.cuda.empty_cache()
    return rec


def gather_section(ctx, name, inst, meta, x, stream_v, off_d, C, nseg, U, rec, checks, headline=False):
    """PCIe transfer mode: rows read zero-copy from pinned host memory (fixed slots
    and packed stream), the uncompressed zero-copy gather of the same rows, the
    measured PCIe ceilings, and the HBM-resident gather (cache mode)."""
    import numpy as np

    import workloads

    torch, ibp, timer, err = ctx.torch, ctx.ibp, ctx.timer, ctx.err
    dev = ctx.dev
    w = inst.w
    S = w.S
    n_rows = inst.data.shape[0]
    row_bytes = inst.row_bytes
    steps = ctx.args.steps if headline else 20
    ids_all = workloads.gather_ids(name, n_rows, steps)
    ids_d = torch.from_numpy(ids_all).to(dev)
    m = ids_all.shape[1]
    step_bytes = m * row_bytes
    out_rows = torch.empty(step_bytes, dtype=torch.uint8, device=dev)
    off_h = off_d.cpu().numpy().view(np.uint64)
    spans = off_h[1:] - off_h[:-1]
    ref_rows = torch.from_numpy(inst.data[ids_all[-1]].reshape(-1).view(np.uint8).copy()).to(dev)
    pcie = ctx.pcie_ceilings()

    def timed(fn):
        fn(0)
        _, ms = timer.run(fn, steps)
        torch.cuda.synchronize()
        return ms

    # fixed slots in pinned host memory (the page's layout for PCIe transfer compression)
    slots_d, flags_d = ibp.ibp_compress_slots(meta, x, S, err=err)
    _, sc_ms = timer.run(lambda i: ibp.ibp_compress_slots(meta, x, S, slots=slots_d, flags=flags_d, err=err), 5)
    slots_h = torch.empty(U, dtype=torch.uint8, pin_memory=True)
    slots_h.copy_(slots_d)
    del slots_d
    s_ms = timed(lambda i: ibp.ibp_decompress_gather_slots(meta, slots_h, flags_d, S, ids_d[i], out=out_rows,
                                                           err=err))
    checks["slots_pinned_gather_equal"] = bool(torch.equal(out_rows, ref_rows))
    n_comp = int(np.unpackbits(flags_d.cpu().numpy().view(np.uint8)).sum())
    used = np.where(spans < S * w.W, (spans + 7) // 8, row_bytes)  # bytes a slot uses
    slot_bytes = sum(int(used[ids].sum()) for ids in ids_all) / steps
    # lines of 128 bytes the used parts touch (host memory is read in 128-byte requests)
    slot_lines = sum(int(((used[ids] + 127) // 128).sum()) for ids in ids_all) / steps
    del slots_h
    log(f"{name}: slot gather from pinned memory {s_ms:.3f} ms")

    # packed stream in pinned host memory, rows located by the offset table in HBM
    host_stream = torch.empty(stream_v.numel(), dtype=torch.uint8, pin_memory=True)
    host_stream.copy_(stream_v)
    p_ms = timed(lambda i: ibp.ibp_decompress_gather(meta, host_stream, off_d, S, ids_d[i], out=out_rows, err=err))
    checks["packed_pinned_gather_equal"] = bool(torch.equal(out_rows, ref_rows))
    packed_bytes = sum(int(((spans[ids] + 7) // 8).sum()) for ids in ids_all) / steps
    first_line = off_h[:-1] // 1024
    last_line = (off_h[1:] + 1023) // 1024
    packed_lines = sum(int((last_line[ids] - first_line[ids]).sum()) for ids in ids_all) / steps
    del host_stream
    log(f"{name}: packed gather from pinned memory {p_ms:.3f} ms")

    # the uncompressed zero-copy gather of the same rows (the transfer IBP replaces)
    raw_host = torch.empty(U, dtype=torch.uint8, pin_memory=True)
    raw_host.copy_(torch.from_numpy(inst.data.reshape(-1).view(np.uint8)))
    r_ms = timed(lambda i: ibp.ibp_gather_raw(raw_host, row_bytes, ids_d[i], out=out_rows, err=err))
    checks["raw_pinned_gather_equal"] = bool(torch.equal(out_rows, ref_rows))
    del raw_host
    raw_lines = step_bytes / 128

    # cache-compression mode: the packed table resident in HBM
    h_ms = timed(lambda i: ibp.ibp_decompress_gather(meta, stream_v, off_d, S, ids_d[i], out=out_rows, err=err))
    checks["hbm_gather_equal"] = bool(torch.equal(out_rows, ref_rows))
    raw_hbm = torch.empty_like(out_rows)
    rh_ms = timed(lambda i: ibp.ibp_gather_raw(x, row_bytes, ids_d[i], out=raw_hbm, err=err))
    del raw_hbm
    h_alg = packed_bytes + 24 * m + step_bytes

    meas = pcie["measured_GBps"]
    rec["step"] = (f"gather of {m} {'Zipf(1.05)' if name == 'dlrm' else 'uniform'} rows ({row_bytes} B each) "
                   "read zero-copy from pinned host memory, fixed-slot layout")
    rec["value"] = step_bytes / s_ms / 1e6
    rec["ms_per_step"] = s_ms
    rec["pcie"] = pcie
    rec["slots_pinned"] = {
        "kernel_ms": s_ms, "effective_GBps": step_bytes / s_ms / 1e6,
        "fraction_of_measured_pcie": step_bytes / s_ms / 1e6 / meas,
        "speedup_vs_uncompressed": r_ms / s_ms, "host_bytes_algorithmic": slot_bytes,
        "host_lines_128B": slot_lines, "rows_compressed": n_comp, "rows": n_rows, "compress_kernel_ms": sc_ms}
    rec["packed_pinned"] = {
        "kernel_ms": p_ms, "effective_GBps": step_bytes / p_ms / 1e6,
        "fraction_of_measured_pcie": step_bytes / p_ms / 1e6 / meas,
        "speedup_vs_uncompressed": r_ms / p_ms, "host_bytes_algorithmic": packed_bytes,
        "host_lines_128B": packed_lines}
    rec["uncompressed_pinned"] = {"kernel_ms": r_ms, "effective_GBps": step_bytes / r_ms / 1e6,
                                  "fraction_of_measured_pcie": step_bytes / r_ms / 1e6 / meas,
                                  "host_lines_128B": raw_lines}
    rec["hbm_cache_mode"] = {
        "kernel_ms": h_ms, "effective_GBps": step_bytes / h_ms / 1e6, "uncompressed_hbm_gather_ms": rh_ms,
        "capacity_gain": U / (C + 8 * (nseg + 1)),
        "roofline": roofline("hbm", h_alg, h_ms, "ibp_decompress_gather, HBM table (decode_kernel)",
                             committed_counters(name, "hbm_gather"))}
    rec["roofline"] = roofline("pcie", slot_bytes, s_ms, "ibp_decompress_gather_slots, pinned slots "
                               "(decode_slots_kernel)", committed_counters(name, "slots_gather"),
                               {"fraction_of_measured_pcie_algorithmic": slot_bytes / s_ms / 1e6 / meas})
    rec["roofline_packed"] = roofline("pcie", packed_bytes, p_ms, "ibp_decompress_gather, pinned packed stream "
                                      "(decode_kernel)", committed_counters(name, "packed_gather"))
    del out_rows, ids_d


def position_metadata_variant(ctx, inst, x, sample, meta, S, rec, checks):
    """Position-dependent metadata (one Mask/Bitval per chunk position of a segment)
    against the single Mask of the same run: ratio, compression and decompression."""
    import numpy as np

    torch, ibp, timer, err = ctx.torch, ctx.ibp, ctx.timer, ctx.err
    dev = ctx.dev
    W, T = inst.w.W, inst.w.T
    U = inst.data.nbytes
    n_chunks = inst.n_chunks
    nseg = ibp.ibp_num_segments(n_chunks, S)
    cap = ibp.ibp_max_stream_bytes(n_chunks, W)
    n_rows_sample = inst.sample.nbytes // (S * W // 8)
    pmeta, _ = ibp.ibp_build_metadata_pos(sample[: n_rows_sample * S * W // 8], W, S, T, counts=False)
    pstream = torch.empty(cap, dtype=torch.uint8, device=dev)
    poff = torch.empty(nseg + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(ibp.ibp_compress_workspace_bytes(n_chunks, S), dtype=torch.uint8, device=dev)
    pcomp = lambda i: ibp.ibp_compress_pos(pmeta, x, err=err, out_stream=pstream, out_offsets=poff, workspace=ws)
    pcomp(0)
    pc_ms = timer.best(pcomp, 10)
    pbits = int(poff[-1].item())
    PC = (pbits + 7) // 8
    pview = pstream[: ibp.ibp_stream_bytes(pbits)]
    pout = torch.empty_like(x)
    pdec = lambda i: ibp.ibp_decompress_pos(pmeta, pview, poff, n_chunks, out=pout, err=err)
    pdec(0)
    pd_ms = timer.best(pdec, 10)
    torch.cuda.synchronize()
    checks["position_metadata_roundtrip_equal"] = bool(torch.equal(pout, x))
    pm = pmeta.mask.cpu().numpy().view(np.uint64)
    pd_alg = PC + 8 * (nseg + 1) + U
    rec["position_metadata"] = {
        "ratio": U / PC, "ratio_single_mask": rec["ratio"]["r_stream"], "positions": S,
        "sample_rows": n_rows_sample, "positions_whose_mask_differs": int((pm != np.uint64(meta.mask)).sum()),
        "compress_kernel_ms": pc_ms, "compress_hbm_fraction": pd_alg / pc_ms / 1e6 / HBM_PEAK_GBPS,
        "decompress_kernel_ms": pd_ms, "decompress_hbm_fraction": pd_alg / pd_ms / 1e6 / HBM_PEAK_GBPS}
    log(f"{inst.w.name}: position metadata ratio {U / PC:.4f} (single Mask {rec['ratio']['r_stream']:.4f}), "
        f"compress {pc_ms:.3f} ms, decompress {pd_ms:.3f} ms")
    del pstream, pout, pview, poff, ws


def zipccl_variant(ctx, inst, x, rec, checks):
    """On a BF16 tensor: the ZipCCL exponent codec, for comparison (not IBP)."""
    torch, ibp, timer, err = ctx.torch, ctx.ibp, ctx.timer, ctx.err
    dev = ctx.dev
    U = inst.data.nbytes
    table = ibp.ibp_zip_table_from_sigma(inst.w.sigma)
    n16 = U // 2
    z = ibp.ibp_zip_compress(table, x, err=err)
    zws = torch.empty(ibp.load_library().ibp_zip_workspace_bytes(n16), dtype=torch.uint8, device=dev)
    zc_ms = timer.best(lambda i: ibp.ibp_zip_compress(table, x, err=err, out=z, workspace=zws), 10)
    E = int(z.eoff[-1].item())
    zout = torch.empty(n16, dtype=torch.int16, device=dev)
    zd_ms = timer.best(lambda i: ibp.ibp_zip_decompress(z, out=zout, err=err), 10)
    torch.cuda.synchronize()
    checks["zipccl_roundtrip_equal"] = bool(torch.equal(zout.view(torch.uint8), x))
    zbytes = n16 + z.codes.numel() + E + z.eoff.numel() * 8
    rec["zipccl_exponent_codec"] = {
        "sigma": inst.w.sigma, "table": list(table), "escape_fraction": E / n16, "ratio": U / zbytes,
        "compress_kernel_ms": zc_ms, "decompress_kernel_ms": zd_ms,
        "decompress_hbm_fraction": (zbytes + U) / zd_ms / 1e6 / HBM_PEAK_GBPS}
    del z, zout, zws


def zero_copy_compress(ctx, meta, inst, x, S, stream_d, off_d, ws, C, rec, checks):
    """Compression in CPU memory: the kernel reads the raw table from pinned host
    memory and writes the stream into pinned host memory (offsets stay in HBM)."""
    import numpy as np

    torch, ibp, timer, err = ctx.torch, ctx.ibp, ctx.timer, ctx.err
    U = inst.data.nbytes
    raw_host = torch.empty(U, dtype=torch.uint8, pin_memory=True)
    raw_host.copy_(torch.from_numpy(inst.data.reshape(-1).view(np.uint8)))
    zc_stream = torch.empty(stream_d.numel(), dtype=torch.uint8, pin_memory=True)
    zc_off = torch.empty_like(off_d)
    zc = lambda i: ibp.ibp_compress(meta, raw_host, S, err=err, out_stream=zc_stream, out_offsets=zc_off, workspace=ws)
    zc(0)
    _, zcc_ms = timer.run(zc, 3)
    torch.cuda.synchronize()
    checks["zero_copy_compress_equal"] = bool(torch.equal(zc_off, off_d)) and \
        bool(torch.equal(zc_stream[:C], stream_d[:C].cpu()))
    rec["compress_zero_copy_host"] = {"kernel_ms": zcc_ms, "pcie_read_GBps": U / zcc_ms / 1e6,
                                      "pcie_write_GBps": C / zcc_ms / 1e6}
    del raw_host, zc_stream, zc_off


def whole_tensor_transfer(ctx, meta, x, stream_v, off_d, n_chunks, S, C, nseg, U, rec, checks):
    """PCIe transfer compression of a whole tensor kept in CPU memory: the decoder reads
    the packed stream zero-copy from pinned host memory and writes the tensor into HBM
    (the offset table, 8 bytes per segment, stays in HBM).  Beside it, the transfers it
    replaces or composes with: hipMemcpyAsync of the raw tensor from pinned memory, and
    hipMemcpyAsync of the stream followed by the device-resident decompression."""
    torch, ibp, timer, err = ctx.torch, ctx.ibp, ctx.timer, ctx.err
    meas = ctx.pcie_ceilings()["measured_GBps"]
    out = torch.empty_like(x)
    host_stream = torch.empty(stream_v.numel(), dtype=torch.uint8, pin_memory=True)
    host_stream.copy_(stream_v)
    zc = lambda i: ibp.ibp_decompress(meta, host_stream, off_d, n_chunks, S, out=out, err=err)
    zc(0)
    zc_ms = timer.best(zc, 2)
    torch.cuda.synchronize()
    checks["pinned_stream_decompress_equal"] = bool(torch.equal(out, x))

    stream_copy = torch.empty_like(stream_v)

    def staged(_i):
        stream_copy.copy_(host_stream, non_blocking=True)
        ibp.ibp_decompress(meta, stream_copy, off_d, n_chunks, S, out=out, err=err)

    staged(0)
    st_ms = timer.best(staged, 2)
    torch.cuda.synchronize()
    checks["staged_stream_decompress_equal"] = bool(torch.equal(out, x))
    del host_stream, stream_copy

    raw_host = torch.empty(U, dtype=torch.uint8, pin_memory=True)
    raw_host.copy_(x)
    raw = lambda i: out.copy_(raw_host, non_blocking=True)
    raw(0)
    raw_ms = timer.best(raw, 2)
    torch.cuda.synchronize()
    checks["raw_h2d_copy_equal"] = bool(torch.equal(out, x))
    del raw_host, out

    host_bytes = C
    rec["whole_tensor_pcie"] = {
        "step": "whole tensor from pinned host memory into HBM, one decoder launch reading the stream zero-copy",
        "zero_copy_decompress_ms": zc_ms, "effective_GBps": U / zc_ms / 1e6,
        "stream_GBps": host_bytes / zc_ms / 1e6,
        "fraction_of_measured_pcie_stream": host_bytes / zc_ms / 1e6 / meas,
        "raw_h2d_copy_ms": raw_ms, "raw_h2d_GBps": U / raw_ms / 1e6,
        "speedup_vs_raw_copy": raw_ms / zc_ms, "latency_change_vs_raw_copy": zc_ms / raw_ms - 1.0,
        "staged_copy_then_decompress_ms": st_ms, "speedup_vs_staged": st_ms / zc_ms,
        "ideal_ms_at_measured_pcie": host_bytes / meas / 1e6,
        "offsets_in_hbm_bytes": 8 * (nseg + 1)}
    log(f"whole tensor over PCIe: zero-copy decompress {zc_ms:.2f} ms, raw copy {raw_ms:.2f} ms, "
        f"staged {st_ms:.2f} ms")


def host_call_cost(ctx) -> dict:
    """Host time of one codec call (argument checks, pointer look-ups, launch set-up,
    enqueue) through the C ABI and through the Python binding: the mean wall time of
    200 calls of ibp_decompress on a small input, queued behind a spin kernel so that
    the GPU never makes the host wait."""
    import ctypes

    torch, ibp = ctx.torch, ctx.ibp
    dev = ctx.dev
    meta = ibp.make_meta(64, 0xFFFFFFFFFF000000, 0)
    x = torch.zeros(64 * 1024, dtype=torch.uint8, device=dev)
    comp = ibp.ibp_compress(meta, x, 256, err=ctx.err)
    out = torch.empty_like(x)
    lib = ibp.load_library()
    args = (ctypes.byref(meta), comp.stream.data_ptr(), comp.stream.numel(), comp.offsets.data_ptr(), comp.n_chunks,
            256, out.data_ptr(), ctx.err.data_ptr(), torch.cuda.current_stream().cuda_stream)
    res = {}
    for label, fn in (("c_abi_us", lambda: lib.ibp_decompress(*args)),
                      ("python_binding_us", lambda: ibp.ibp_decompress(meta, comp.stream, comp.offsets, comp.n_chunks,
                                                                       256, out=out, err=ctx.err))):
        torch.cuda.synchronize()
        ctx.timer._hold(50.0)
        t0 = time.perf_counter()
        for _ in range(200):
            fn()
        res[label] = (time.perf_counter() - t0) / 200 * 1e6
        torch.cuda.synchronize()
    return res


# ---------------------------------------------------------------------------- CPU oracle baseline

def _pool_map(fn, items, threads):
    if threads == 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def _ranges(n, parts):
    b = [n * i // parts for i in range(parts + 1)]
    return [(b[i], b[i + 1]) for i in range(parts) if b[i + 1] > b[i]]


def _stitch(parts, total_bits, threads):
    """Bit-level concatenation of byte buffers holding parts[i] = (buf, nbits), in
    parallel: each part writes the bytes only it covers; the bytes two parts share
    are OR-ed afterwards."""
    import numpy as np

    out = np.zeros((total_bits + 7) // 8 + 1, np.uint8)
    bases = []
    b = 0
    for _, nb in parts:
        bases.append(b)
        b += nb
    shared = []

    def one(i):
        buf, nb = parts[i]
        n = (nb + 7) // 8
        if n == 0:
            return
        b0, sh = bases[i] // 8, bases[i] % 8
        wide = buf[:n].astype(np.uint16) << sh
        lo = (wide & 0xFF).astype(np.uint8)
        hi = (wide >> 8).astype(np.uint8)
        # byte b0 + j (1 <= j < n) = lo[j] | hi[j - 1]; byte b0 and byte b0 + n are shared
        out[b0 + 1:b0 + n] = lo[1:] | hi[:-1]
        shared.append((b0, lo[0]))
        shared.append((b0 + n, hi[-1]))

    _pool_map(one, range(len(parts)), threads)
    for pos, v in shared:
        out[pos] |= v
    return out[: (total_bits + 7) // 8]


def cpu_baseline(inst, meta, stream_d, off_d, gpu_bits, gpu_counts, budget_s, checks):
    """The oracle on the host's cores, 1 thread and N threads, on bounded samples of
    this workload: metadata over the workload's whole metadata sample, compression of
    the first segments (rows), and decompression of the oracle's own stream of them
    (for gather workloads: a gather of those rows in a seeded random order).  The
    oracle's results are compared with the GPU's on the same samples."""
    import ctypes

    import numpy as np

    import oracle

    L = oracle.lib()
    N = cpu_threads()
    w = inst.w
    W, T, S = w.W, w.T, w.S
    cb = W // 8
    u64 = ctypes.c_uint64
    mask, bitval = meta.mask, meta.bitval
    data = inst.data.reshape(-1).view(np.uint8)
    res = {"cores": N, "nproc": os.cpu_count(), "cpu_model": cpu_model(), "kind": "oracle", "unit": "GB/s",
           "ops": {}}

    # --- metadata: count ones over the sample (N ranges), then the threshold rule
    smp = np.ascontiguousarray(inst.sample.reshape(-1).view(np.uint8))
    ns = smp.size // cb

    def count(r):
        c1 = np.zeros(64, np.uint64)
        rc = L.ibpo_count_ones(smp.ctypes.data + r[0] * cb, 1, r[1] - r[0], W, c1.ctypes.data)
        assert rc == 0
        return c1

    def meta_run(threads):
        t0 = time.perf_counter()
        c = sum(_pool_map(count, _ranges(ns, threads), threads))
        mk, bv = u64(0), u64(0)
        cc = np.ascontiguousarray(c, np.uint64)
        rc = L.ibpo_meta_from_counts(cc.ctypes.data, ns, W, T, ctypes.byref(mk), ctypes.byref(bv))
        assert rc == 0
        return time.perf_counter() - t0, (mk.value, bv.value, cc[:W].tolist())

    t1, r1 = meta_run(1)
    tn, rn = meta_run(N)
    checks["oracle_metadata_equal"] = r1 == rn == (mask, bitval, list(gpu_counts))
    res["ops"]["metadata"] = {"bytes": smp.size, "t1_s": t1, "tN_s": tn, "t1_GBps": smp.size / t1 / 1e9,
                              "tN_GBps": smp.size / tn / 1e9,
                              "sample": f"the whole metadata sample, {ns} chunks"}

    # --- compression of the first segments
    nseg_all = (inst.n_chunks + S - 1) // S
    seg_bytes = S * cb

    def encode_range(r):
        k0, k1 = r
        n = min(k1 * S, inst.n_chunks) - k0 * S
        off = np.zeros(k1 - k0 + 1, np.uint64)
        buf = np.zeros((n * (W + 1) + 7) // 8 + 1, np.uint8)
        rc = L.ibpo_encode(data.ctypes.data + k0 * seg_bytes, 1, n, W, mask, bitval, S, off.ctypes.data,
                           buf.ctypes.data, buf.size)
        assert rc == 0
        return buf, off

    def compress_run(ksegs, threads):
        t0 = time.perf_counter()
        parts = _pool_map(encode_range, _ranges(ksegs, 1 if threads == 1 else threads * 4), threads)
        bits = [int(o[-1]) for _, o in parts]
        stream = _stitch([(b, nb) for (b, _), nb in zip(parts, bits)], sum(bits), threads)
        offs, base = [np.zeros(1, np.uint64)], 0
        for (_, o), nb in zip(parts, bits):
            offs.append(o[1:] + np.uint64(base))
            base += nb
        off = np.concatenate(offs)
        return time.perf_counter() - t0, stream, off

    # size the samples from a short calibration run: about budget_s each
    kcal = max(1, min(nseg_all, (1 << 20) // seg_bytes))
    tc, _, _ = compress_run(kcal, 1)
    rate = kcal / max(tc, 1e-6)
    k1 = int(max(1, min(nseg_all, rate * budget_s)))
    kN = int(max(1, min(nseg_all, k1 * N)))
    t1, s1, o1 = compress_run(k1, 1)
    tn, sn, on = compress_run(kN, N)
    # the GPU's stream and offsets of the same segments
    g_off = off_d[: kN + 1].cpu().numpy().view(np.uint64)
    nb = (int(g_off[-1]) + 7) // 8
    g_stream = stream_d[:nb].cpu().numpy()
    tail = int(g_off[-1]) % 8
    if tail:
        g_stream = g_stream.copy()
        g_stream[-1] &= (1 << tail) - 1  # the next segment's bits share the last byte
    checks["oracle_compress_equal"] = bool(np.array_equal(on, g_off) and np.array_equal(sn, g_stream)
                                           and np.array_equal(o1, on[: k1 + 1])
                                           and np.array_equal(s1[: int(o1[-1]) // 8], sn[: int(o1[-1]) // 8]))
    b1, bN = min(k1 * S, inst.n_chunks) * cb, min(kN * S, inst.n_chunks) * cb
    res["ops"]["compress"] = {"t1_s": t1, "tN_s": tn, "t1_GBps": b1 / t1 / 1e9, "tN_GBps": bN / tn / 1e9,
                              "sample": f"first {k1} segments ({b1} B) on 1 thread, first {kN} ({bN} B) on {N}"}
    del g_stream

    # --- decompression of the oracle's own stream
    sn_c = np.ascontiguousarray(sn)
    if inst.w.gather:
        rng = np.random.default_rng(w.seed)
        order = rng.permutation(kN).astype(np.int64)

        def gather_run(nids, threads):
            out = np.zeros(nids * seg_bytes, np.uint8)

            def one(r):
                a, b = r
                rc = L.ibpo_decode_gather(sn_c.ctypes.data, sn_c.size, on.ctypes.data, kN, S,
                                          order.ctypes.data + 8 * a, b - a, W, mask, bitval,
                                          out.ctypes.data + a * seg_bytes, 1)
                assert rc == 0

            t0 = time.perf_counter()
            _pool_map(one, _ranges(nids, threads * 4), threads)
            return time.perf_counter() - t0, out

        n1 = min(k1, kN)
        t1, d1 = gather_run(n1, 1)
        tn, dn = gather_run(kN, N)
        ref = data[: kN * seg_bytes].reshape(kN, seg_bytes)[order]
        checks["oracle_decompress_equal"] = bool(np.array_equal(dn.reshape(kN, -1), ref)
                                                 and np.array_equal(d1.reshape(n1, -1), ref[:n1]))
        res["ops"]["decompress"] = {
            "t1_s": t1, "tN_s": tn, "t1_GBps": d1.size / t1 / 1e9, "tN_GBps": dn.size / tn / 1e9,
            "sample": (f"gather of {n1} (1 thread) and {kN} ({N} threads) rows, seeded random order, from the "
                       f"oracle's stream of the first {kN} rows")}
    else:
        def decode_run(ksegs, threads):
            nb_out = min(ksegs * S, inst.n_chunks) * cb
            out = np.zeros(nb_out, np.uint8)

            def one(r):
                a, b = r
                n = min(b * S, inst.n_chunks) - a * S
                rc = L.ibpo_decode(sn_c.ctypes.data, sn_c.size, on.ctypes.data + 8 * a, n, W, mask, bitval, S,
                                   out.ctypes.data + a * seg_bytes, 1)
                assert rc == 0

            t0 = time.perf_counter()
            _pool_map(one, _ranges(ksegs, threads * 4), threads)
            return time.perf_counter() - t0, out

        t1, d1 = decode_run(k1, 1)
        tn, dn = decode_run(kN, N)
        checks["oracle_decompress_equal"] = bool(np.array_equal(dn, data[: dn.size])
                                                 and np.array_equal(d1, data[: d1.size]))
        res["ops"]["decompress"] = {"t1_s": t1, "tN_s": tn, "t1_GBps": d1.size / t1 / 1e9,
                                    "tN_GBps": dn.size / tn / 1e9,
                                    "sample": f"first {k1} segments on 1 thread, first {kN} on {N}"}
    d = res["ops"]["decompress"]
    res["value"] = d["tN_GBps"]
    res["single_thread_GBps"] = d["t1_GBps"]
    res["sample"] = (f"oracle decompression on {N} threads: {d['sample']}; metadata and compression figures "
                     f"under ops")
    return res


# ---------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default=",".join(CONFIG_ORDER),
                    help="workloads to run, in order (tiny,gnn,dlrm,llm,ids; variants: sparse,llm16,mixed)")
    ap.add_argument("--headline", default=None,
                    help="the workload whose step is timed K times (default: ids when it runs, else the first)")
    ap.add_argument("--variants", action="store_true", help="also run the sparse, W = 16 and mixed feature-row variants")
    ap.add_argument("--scale", type=float, default=1.0, help="shrink every workload (testing only)")
    ap.add_argument("--cpu-seconds", type=float, default=0.5, help="oracle time per operation on one thread")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the IBP hot path has no "
              "cross-GPU step; the sharding plan is described in the design notes.", file=sys.stderr)
        return 2
    names = [n for n in args.configs.split(",") if n]
    if args.variants:
        names += [v for v in VARIANTS if v not in names]
    if args.headline is None:
        args.headline = "ids" if "ids" in names else names[0]
    if args.headline not in names:
        names.append(args.headline)
    import workloads
    for n in names:
        if n not in workloads.WORKLOADS:
            print(f"unknown workload {n}", file=sys.stderr)
            return 2

    ctx = Ctx(args)
    log("start")
    results = {}
    for n in names:
        results[n] = run_workload(ctx, n, headline=(n == args.headline))
    dc = ctx.device_copy()
    host_call = host_call_cost(ctx)
    # a plain device copy of known size (the last one of the run): its counter readings
    # calibrate FETCH_SIZE / WRITE_SIZE in the committed counter summaries
    cal = ctx.torch.empty(256 << 20, dtype=ctx.torch.uint8, device=ctx.dev)
    cal2 = ctx.torch.empty_like(cal)
    cal2.copy_(cal)
    ctx.torch.cuda.synchronize()
    del cal, cal2

    head = results[args.headline]
    w = workloads.WORKLOADS[args.headline]
    all_checks = {f"{n}.{k}": v for n, r in results.items() for k, v in r["checks"].items()}
    err_words = {n: r["device_error_word"] for n, r in results.items()}
    configs = {n: results[n] for n in names if n in CONFIG_ORDER}
    variants = {n: results[n] for n in names if n not in CONFIG_ORDER}
    line = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"u{w.W}", "data": "synthetic (seeded SplitMix64 generators)",
        "config": {"workload": head["workload"], "elements": head["elements"],
                   "W": w.W, "T": w.T, "S": w.S,
                   "source": "pinned host memory, fixed slots" if w.gather else "compressed stream resident in HBM",
                   "step": head["step"]},
        "compression_ratio": head["ratio"]["r_stream"], "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "configs": configs, "variants": variants, "device_copy_reference": dc, "host_call_cost": host_call,
        "checks": {"all_equal": all(all_checks.values()), **all_checks}, "device_error_words": err_words,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)
    log("done")
    return 0 if all(all_checks.values()) and not any(err_words.values()) else 1


if __name__ == "__main__":
    sys.exit(main())
