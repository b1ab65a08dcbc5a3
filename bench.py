"""Benchmark of the IBP codec on one MI355X; prints one JSON line.

A step is one pass of the hot path over one batch of the workload:

* gnn (default) and dlrm: a gather of 65,536 uniform (gnn) or 32,768 Zipf(1.05)
  (dlrm) row ids, each row one compressed segment, decoded into HBM.  ``value``
  is measured with the compressed table resident in HBM; the same gathers read
  zero-copy from pinned host memory over PCIe are measured in the same run and
  reported under ``pcie_sourced``, beside the measured PCIe ceilings and the
  uncompressed zero-copy gather they replace.
* tiny, llm, ids: a device-resident decompression of the whole tensor.

Metadata (step 1) and compression (step 2) run first on the same data and are
timed and reported too, and the decoded output is compared against the input.
``cpu_baseline`` is the CPU oracle (one thread) on a bounded sample of the same
work.  ``roofline`` is for the kernel of the timed step: its algorithmic bytes
per launch over its mean launch time (HIP events on its stream).  ``traffic``
comes from the committed rocprofv3 counter summary of that kernel, and is null
when the kernel source has changed since the counters were taken.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IBP decompress effective GB/s (HBM- and PCIe-sourced) + compression ratio"
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E, AMD published
PCIE_PEAK_GBPS = 64.0      # PCIe 5.0 x16, one direction, published link rate
KERNEL_SOURCES = [os.path.join(ROOT, "bit_packing_amd", "csrc", f) for f in
                  ("ibp_device.h", "ibp_decode_loops.h", "ibp_internal.h", "ibp_meta.hip", "ibp_encode.hip",
                   "ibp_decode.hip", "ibp_decode_pos.hip", "ibp_slots.hip", "ibp_zip.hip")]


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


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/<kernel>_<workload>_traffic.txt, if that summary
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
        """Per-launch milliseconds of the fastest of `runs` timed regions of n launches
        (for the side measurements; the timed step uses one region of exactly K steps)."""
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gnn", choices=["gnn", "dlrm", "tiny", "llm", "ids", "sparse", "llm16"])
    ap.add_argument("--scale", type=float, default=1.0, help="shrink the workload (testing only)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the IBP hot path has no "
              "cross-GPU step; the sharding plan is described in the design notes.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_packing_amd as ibp
    import workloads

    ibp.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    inst = workloads.generate(args.workload, args.scale)
    W, T, S = w.W, w.T, w.S
    n_chunks = inst.n_chunks
    U = inst.data.nbytes
    gather = w.gather > 0
    extra = {}

    x = torch.from_numpy(inst.data.reshape(-1).view(np.uint8)).to(dev)
    sample = torch.from_numpy(inst.sample.reshape(-1).view(np.uint8)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    timer = Timer(torch)

    # ---- step 1: metadata (synchronous by definition; wall time)
    meta, _ = ibp.ibp_build_metadata(sample, W, T)
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        meta, _ = ibp.ibp_build_metadata(sample, W, T)
    extra["metadata"] = {"ms": (time.perf_counter() - t0) / reps * 1e3, "sample_chunks": int(inst.sample.nbytes * 8 // W),
                         "mask": hex(meta.mask), "bitval": hex(meta.bitval)}

    # ---- step 2: compression, HBM -> HBM
    cap = ibp.ibp_max_stream_bytes(n_chunks, W)
    stream_d = torch.empty(cap, dtype=torch.uint8, device=dev)
    nseg = ibp.ibp_num_segments(n_chunks, S)
    off_d = torch.empty(nseg + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(ibp.ibp_compress_workspace_bytes(n_chunks, S), dtype=torch.uint8, device=dev)

    def compress(_i):
        ibp.ibp_compress(meta, x, S, err=err, out_stream=stream_d, out_offsets=off_d, workspace=ws)

    compress(0)
    creps = 10 if U > (64 << 20) else 20
    c_ms = timer.best(compress, creps)
    total_bits = int(off_d[-1].item())
    C = (total_bits + 7) // 8
    r_stream = U / C
    r_total = U / (C + 8 * (nseg + 1) + 24)
    extra["compress"] = {"kernel_ms": c_ms, "effective_GBps": U / c_ms / 1e6,
                         "algorithmic_GBps": (U + C + 8 * (nseg + 1)) / c_ms / 1e6}
    extra["ratio"] = {"r_stream": r_stream, "r_total": r_total, "stream_bytes": C, "input_bytes": U,
                      "segments": nseg, "S": S}
    stream_bytes = ibp.ibp_stream_bytes(total_bits)
    stream_d = stream_d[:stream_bytes]

    # ---- step 3: device-resident decompression of the whole tensor
    out_full = torch.empty_like(x)

    def decompress(_i):
        ibp.ibp_decompress(meta, stream_d, off_d, n_chunks, S, out=out_full, err=err)

    decompress(0)
    dreps = 10 if U > (64 << 20) else 20
    d_ms = timer.best(decompress, dreps)
    d_alg = C + 8 * (nseg + 1) + U
    extra["decompress_device"] = {"kernel_ms": d_ms, "effective_GBps": U / d_ms / 1e6,
                                  "algorithmic_GBps": d_alg / d_ms / 1e6,
                                  "hbm_fraction": d_alg / d_ms / 1e6 / HBM_PEAK_GBPS}
    torch.cuda.synchronize()
    roundtrip_ok = bool(torch.equal(out_full, x))
    del out_full

    # ---- variant: position-dependent metadata (one Mask/Bitval per chunk position
    # of a segment), built from the same sample taken as rows of S chunks
    pos_ok = None
    n_rows_sample = inst.sample.nbytes // (S * W // 8)
    if n_rows_sample >= 1:
        pmeta, _ = ibp.ibp_build_metadata_pos(sample[: n_rows_sample * S * W // 8], W, S, T, counts=False)
        pstream = torch.empty(cap, dtype=torch.uint8, device=dev)
        poff = torch.empty_like(off_d)
        pcomp = lambda i: ibp.ibp_compress_pos(pmeta, x, err=err, out_stream=pstream, out_offsets=poff, workspace=ws)
        pcomp(0)
        pc_ms = timer.best(pcomp, creps)
        pbits = int(poff[-1].item())
        PC = (pbits + 7) // 8
        pview = pstream[: ibp.ibp_stream_bytes(pbits)]
        pout = torch.empty_like(x)
        pdec = lambda i: ibp.ibp_decompress_pos(pmeta, pview, poff, n_chunks, out=pout, err=err)
        pdec(0)
        pd_ms = timer.best(pdec, dreps)
        torch.cuda.synchronize()
        pos_ok = bool(torch.equal(pout, x))
        pm = pmeta.mask.cpu().numpy().view(np.uint64)
        pd_alg = PC + 8 * (nseg + 1) + U
        extra["position_metadata"] = {
            "ratio": U / PC, "ratio_single_mask": r_stream, "positions": S, "sample_rows": n_rows_sample,
            "positions_whose_mask_differs": int((pm != np.uint64(meta.mask)).sum()),
            "compress_kernel_ms": pc_ms, "decompress_kernel_ms": pd_ms,
            "decompress_algorithmic_GBps": pd_alg / pd_ms / 1e6, "hbm_fraction": pd_alg / pd_ms / 1e6 / HBM_PEAK_GBPS,
            "parity_ok": pos_ok}
        del pstream, pout, pview

    # ---- comparison codec on BF16 tensors: exponent coding as on the ZipCCL page,
    # with the exponent table derived from the distribution's sigma (no histogram)
    zip_ok = None
    if w.dtype == "uint16" and w.sigma:
        table = ibp.ibp_zip_table_from_sigma(w.sigma)
        n16 = U // 2
        z = ibp.ibp_zip_compress(table, x, err=err)
        zws = torch.empty(ibp.load_library().ibp_zip_workspace_bytes(n16), dtype=torch.uint8, device=dev)
        zc_ms = timer.best(lambda i: ibp.ibp_zip_compress(table, x, err=err, out=z, workspace=zws), creps)
        E = int(z.eoff[-1].item())
        zout = torch.empty(n16, dtype=torch.int16, device=dev)
        zd_ms = timer.best(lambda i: ibp.ibp_zip_decompress(z, out=zout, err=err), dreps)
        torch.cuda.synchronize()
        zip_ok = bool(torch.equal(zout.view(torch.uint8), x))
        zbytes = n16 + z.codes.numel() + E + z.eoff.numel() * 8
        z_alg = zbytes + U
        extra["zipccl_exponent_codec"] = {
            "sigma": w.sigma, "table": list(table), "escapes": E, "escape_fraction": E / n16,
            "ratio": U / zbytes, "ratio_ibp": r_stream, "compress_kernel_ms": zc_ms, "decompress_kernel_ms": zd_ms,
            "decompress_algorithmic_GBps": z_alg / zd_ms / 1e6, "decompress_hbm_fraction": z_alg / zd_ms / 1e6 / HBM_PEAK_GBPS,
            "compress_algorithmic_GBps": z_alg / zc_ms / 1e6, "parity_ok": zip_ok}
        del z, zout, zws

    off_h = off_d.cpu().numpy().view(np.uint64)
    if gather:
        n_rows = inst.data.shape[0]
        row_bytes = inst.row_bytes
        ids_all = workloads.gather_ids(args.workload, n_rows, args.warmup + args.steps)
        ids_d = torch.from_numpy(ids_all).to(dev)
        m = ids_all.shape[1]
        out_rows = torch.empty(m * row_bytes, dtype=torch.uint8, device=dev)
        spans = (off_h[1:] - off_h[:-1])
        # algorithmic bytes per gather: the rows' compressed spans, two offsets and an id per row, the output
        alg_hbm = [int(((spans[ids] + 7) // 8).sum()) + 24 * m + m * row_bytes for ids in ids_all]
        pcie_bytes = [int(((spans[ids] + 7) // 8).sum()) for ids in ids_all]

        def gather_from(src):
            def fn(i):
                ibp.ibp_decompress_gather(meta, src, off_d, S, ids_d[i], out=out_rows, err=err)
            return fn

        # timed step: gather from the HBM-resident compressed table
        step = gather_from(stream_d)
        for i in range(args.warmup):
            step(i)
        # kernel durations: HIP events around each launch of an eager pass
        eager_wall, k_ms = timer.run(lambda i: step(args.warmup + i), args.steps)
        # whole-step throughput: the same K launches replayed from a HIP graph
        wall = graph_wall(torch, step, args.warmup, args.steps)
        extra["timed_step"] = {"graph_ms_per_step": wall / args.steps * 1e3,
                               "eager_queued_ms_per_step": eager_wall / args.steps * 1e3}
        last = ids_all[-1]
        ref_rows = torch.from_numpy(inst.data.reshape(n_rows, -1)[last].reshape(-1).view(np.uint8).copy()).to(dev)
        gather_ok = bool(torch.equal(out_rows, ref_rows))
        # the same rows gathered uncompressed from the HBM copy of the table (context for the roofline)
        raw_rows = torch.empty_like(out_rows)
        _, rawd_ms = timer.run(lambda i: ibp.ibp_gather_raw(x, row_bytes, ids_d[args.warmup + i], out=raw_rows), args.steps)
        extra["uncompressed_hbm_gather"] = {"kernel_ms": rawd_ms, "effective_GBps": m * row_bytes / rawd_ms / 1e6,
                                            "algorithmic_GBps": (2 * m * row_bytes + 8 * m) / rawd_ms / 1e6}
        del raw_rows
        step_bytes = m * row_bytes
        value = step_bytes * args.steps / wall / 1e9
        ms_per_step = wall / args.steps * 1e3
        achieved = (sum(alg_hbm[args.warmup:]) / args.steps) / k_ms / 1e6
        kernel_name, kernel_label = "decode_kernel_gather", "ibp_decompress_gather (HBM-resident table)"
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": committed_traffic(kernel_name, args.workload),
                    "kernel": kernel_label, "kernel_ms": k_ms,
                    "algorithmic_bytes_per_launch": sum(alg_hbm[args.warmup:]) / args.steps}

        # the same gathers with the compressed table in pinned host memory (zero-copy PCIe)
        host_stream = torch.empty(stream_bytes, dtype=torch.uint8, pin_memory=True)
        host_stream.copy_(stream_d)
        hstep = gather_from(host_stream)
        for i in range(args.warmup):
            hstep(i)
        h_wall, h_ms = timer.run(lambda i: hstep(args.warmup + i), args.steps)
        h_ok = bool(torch.equal(out_rows, ref_rows))
        # PCIe ceilings measured in this run: hipMemcpyAsync H2D, and a zero-copy streaming read
        probe = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
        probe_d = torch.empty_like(probe, device=dev)
        _, cp_ms = timer.run(lambda i: probe_d.copy_(probe, non_blocking=True), 5)
        seq = torch.arange((256 << 20) // 4096, dtype=torch.int64, device=dev)
        _, zc_ms = timer.run(lambda i: ibp.ibp_gather_raw(probe, 4096, seq, out=probe_d), 5)
        pcie_meas = max(probe.numel() / cp_ms / 1e6, probe.numel() / zc_ms / 1e6)
        # uncompressed zero-copy gather of the same rows (the transfer IBP replaces)
        raw_host = torch.empty(U, dtype=torch.uint8, pin_memory=True)
        raw_host.copy_(torch.from_numpy(inst.data.reshape(-1).view(np.uint8)))
        _, raw_ms = timer.run(lambda i: ibp.ibp_gather_raw(raw_host, row_bytes, ids_d[args.warmup + i],
                                                           out=out_rows), args.steps)
        # zero-copy compression in CPU memory: the kernel reads the raw table from pinned
        # host memory and writes the stream into pinned host memory (offsets stay in HBM)
        zc_stream = torch.empty(cap, dtype=torch.uint8, pin_memory=True)
        zc_off = torch.empty_like(off_d)
        zc = lambda i: ibp.ibp_compress(meta, raw_host, S, err=err, out_stream=zc_stream, out_offsets=zc_off,
                                        workspace=ws)
        zc(0)
        _, zcc_ms = timer.run(zc, 3)
        torch.cuda.synchronize()
        zc_ok = bool(torch.equal(zc_off, off_d)) and bool(torch.equal(zc_stream[:C], stream_d[:C].cpu()))
        extra["compress_zero_copy_host"] = {"kernel_ms": zcc_ms, "effective_GBps": U / zcc_ms / 1e6,
                                            "pcie_read_GBps": U / zcc_ms / 1e6, "pcie_write_GBps": C / zcc_ms / 1e6,
                                            "parity_ok": zc_ok}
        # fixed-slot (in-place) layout of the same table: compress into slots in HBM,
        # copy them to pinned host memory, gather the same rows from there
        slots_d, flags_d = ibp.ibp_compress_slots(meta, x, S, err=err)
        _, sc_ms = timer.run(lambda i: ibp.ibp_compress_slots(meta, x, S, slots=slots_d, flags=flags_d, err=err), 5)
        slots_h = torch.empty(U, dtype=torch.uint8, pin_memory=True)
        slots_h.copy_(slots_d)
        slot_rows = torch.empty_like(out_rows)
        sstep = lambda i: ibp.ibp_decompress_gather_slots(meta, slots_h, flags_d, S, ids_d[args.warmup + i],
                                                          out=slot_rows, err=err)
        sstep(0)
        _, sg_ms = timer.run(sstep, args.steps)
        torch.cuda.synchronize()
        slots_ok = bool(torch.equal(slot_rows, ref_rows))
        n_comp = int(np.unpackbits(flags_d.cpu().numpy().view(np.uint8)).sum())
        # a slot row is read up to its used length: the segment's bits when it compresses, else the raw row
        used = np.where(spans < S * W, (spans + 7) // 8, row_bytes)
        sb = sum(int(used[ids].sum()) for ids in ids_all[args.warmup:]) / args.steps
        extra["slots_pinned"] = {"effective_GBps": step_bytes / sg_ms / 1e6, "kernel_ms": sg_ms,
                                 "pcie_read_GBps_algorithmic": sb / sg_ms / 1e6,
                                 "fraction_of_measured_pcie": step_bytes / sg_ms / 1e6 / pcie_meas,
                                 "speedup_vs_uncompressed": raw_ms / sg_ms, "speedup_vs_packed": h_ms / sg_ms,
                                 "compress_kernel_ms": sc_ms, "rows_compressed": n_comp, "rows": n_rows,
                                 "parity_ok": slots_ok}
        del slots_d, slots_h, slot_rows
        del probe, probe_d, raw_host, zc_stream, zc_off
        # cache-compression mode: rows an HBM cache of fixed size holds, compressed vs raw
        extra["cache_mode"] = {"capacity_gain": U / (C + 8 * (nseg + 1)),
                               "rows_per_GiB_raw": (1 << 30) / row_bytes,
                               "rows_per_GiB_compressed": (1 << 30) * n_rows / (C + 8 * (nseg + 1))}
        pb = sum(pcie_bytes[args.warmup:]) / args.steps
        extra["pcie_sourced"] = {
            "effective_GBps": step_bytes / h_ms / 1e6, "kernel_ms": h_ms, "queued_ms_per_step": h_wall / args.steps * 1e3,
            "pcie_read_GBps_algorithmic": pb / h_ms / 1e6,
            "pcie_measured_GBps": pcie_meas, "memcpy_h2d_GBps": (256 << 20) / cp_ms / 1e6,
            "zero_copy_stream_GBps": (256 << 20) / zc_ms / 1e6,
            "fraction_of_measured_pcie": step_bytes / h_ms / 1e6 / pcie_meas,
            "uncompressed_zero_copy_gather_GBps": step_bytes / raw_ms / 1e6,
            "speedup_vs_uncompressed": raw_ms / h_ms,
            "roofline": {"bound": "pcie", "achieved": pb / h_ms / 1e6, "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                         "frac": pb / h_ms / 1e6 / PCIE_PEAK_GBPS},
            "parity_ok": h_ok}
        del host_stream
        checks = {"roundtrip_equal": roundtrip_ok, "gather_equal": gather_ok, "pcie_gather_equal": h_ok,
                  "zero_copy_compress_equal": zc_ok, "slots_gather_equal": slots_ok}
        config = {"workload": f"{args.workload}: {w.description}", "rows": n_rows, "row_bytes": row_bytes,
                  "W": W, "T": T, "S": S, "ids_per_step": m,
                  "ids": "Zipf(1.05)" if args.workload == "dlrm" else "uniform",
                  "source": "compressed table resident in HBM"}
        cpu_work = ("gather", ids_all[args.warmup:].reshape(-1), row_bytes)
    else:
        out_full = torch.empty_like(x)

        def step(i):
            ibp.ibp_decompress(meta, stream_d, off_d, n_chunks, S, out=out_full, err=err)

        for i in range(args.warmup):
            step(i)
        eager_wall, k_ms = timer.run(step, args.steps)
        wall = graph_wall(torch, step, 0, args.steps)
        extra["timed_step"] = {"graph_ms_per_step": wall / args.steps * 1e3,
                               "eager_queued_ms_per_step": eager_wall / args.steps * 1e3}
        value = U * args.steps / wall / 1e9
        ms_per_step = wall / args.steps * 1e3
        achieved = d_alg / k_ms / 1e6
        kernel_name = "decode_kernel"
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": committed_traffic(kernel_name, args.workload),
                    "kernel": "ibp_decompress", "kernel_ms": k_ms, "algorithmic_bytes_per_launch": d_alg}
        torch.cuda.synchronize()
        checks = {"roundtrip_equal": bool(torch.equal(out_full, x)) and roundtrip_ok}
        config = {"workload": f"{args.workload}: {w.description}", "elements": int(inst.data.size),
                  "W": W, "T": T, "S": S, "source": "compressed stream resident in HBM"}
        cpu_work = ("decode", None, None)
    if pos_ok is not None:
        checks["position_metadata_roundtrip"] = pos_ok
    if zip_ok is not None:
        checks["zipccl_roundtrip"] = zip_ok
    torch.cuda.synchronize()
    errword = int(err.item())

    # reference ceiling for kernels that read and write HBM: a plain 256 MiB device copy
    ref_a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    ref_b = torch.empty_like(ref_a)
    _, dc_ms = timer.run(lambda i: ref_b.copy_(ref_a), 10)
    extra["device_copy_reference"] = {"GBps": 2 * (256 << 20) / dc_ms / 1e6,
                                      "fraction_of_peak": 2 * (256 << 20) / dc_ms / 1e6 / HBM_PEAK_GBPS}
    del ref_a, ref_b
    # a plain device copy of known size (the last one of the run): its counter readings
    # calibrate FETCH_SIZE / WRITE_SIZE
    cal = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()
    del cal, cal2

    # the counter traffic of the step kernel as a rate, beside the device copy's
    # (how close the kernel moves its actual bytes to what a plain copy achieves)
    if roofline["bound"] == "hbm" and roofline["traffic"]:
        tr_gbps = roofline["traffic"] / roofline["kernel_ms"] / 1e6
        roofline["traffic_GBps"] = tr_gbps
        roofline["traffic_rate_vs_device_copy"] = tr_gbps / extra["device_copy_reference"]["GBps"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inst, meta, stream_d, off_h, S, cpu_work, args.cpu_seconds)

    res = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"u{W}", "data": "synthetic (seeded SplitMix64 generators)",
        "config": config, "compression_ratio": r_stream, "roofline": roofline, "cpu_baseline": cpu,
        "checks": {**checks, "device_error_word": errword}, "extra": extra,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(res), flush=True)
    return 0 if all(checks.values()) and errword == 0 else 1


def cpu_baseline(inst, meta, stream_d, off_h, S, work, budget_s):
    """The oracle, one thread, on a bounded sample of the same work."""
    import numpy as np

    import oracle

    stream_h = stream_d.cpu().numpy()
    W = inst.w.W
    kind, ids, row_bytes = work
    t0 = time.perf_counter()
    done = 0
    if kind == "gather":
        for start in range(0, len(ids), 1024):
            oracle.decode_gather(stream_h, off_h, S, ids[start:start + 1024], W, meta.mask, meta.bitval, np.uint8)
            done += min(1024, len(ids) - start)
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
        nbytes = done * row_bytes
        sample = f"oracle gather of the first {done} row ids of the timed steps ({nbytes} bytes out)"
    else:
        nseg = len(off_h) - 1
        seg_bytes = S * W // 8
        k = 0
        while k < nseg and time.perf_counter() - t0 < budget_s:
            kk = min(nseg, k + 256)
            last_chunks = min(kk * S, inst.n_chunks) - k * S
            sub_off = (off_h[k:kk + 1] - off_h[k]).astype(np.uint64)
            b0 = int(off_h[k]) // 8
            shift = int(off_h[k]) % 8
            # re-base the segment range to a byte boundary for the oracle
            seg = np.unpackbits(stream_h[b0:(int(off_h[kk]) + 7) // 8 + 1], bitorder="little")[shift:]
            sub_stream = np.packbits(seg, bitorder="little")
            oracle.decode(sub_stream, sub_off, last_chunks, W, meta.mask, meta.bitval, S, np.uint8)
            done += last_chunks
            k = kk
        el = time.perf_counter() - t0
        nbytes = done * W // 8
        sample = f"oracle decode of the first {k} segments ({nbytes} bytes out)"
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": sample,
            "seconds": el}


if __name__ == "__main__":
    sys.exit(main())
