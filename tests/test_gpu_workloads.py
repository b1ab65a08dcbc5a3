"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times (same W, T, S, same calls).

At these sizes the oracle cannot encode everything in seconds, so it checks:
the metadata (all counts), the whole offset table (the oracle's size pass is
cheap), sampled segments bit for bit (the oracle encodes single segments), and
the round trip and the gathers against the input itself.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _bits(buf: np.ndarray, a: int, b: int) -> np.ndarray:
    """Stream bits [a, b) of a byte buffer."""
    chunk = buf[a // 8:(b + 7) // 8]
    return np.unpackbits(chunk, bitorder="little")[a % 8:a % 8 + (b - a)]


@pytest.mark.parametrize("name", ["tiny", "gnn", "dlrm", "llm", "ids", "sparse", "llm16", "mixed"])
def test_workload_full_size(name):
    import bit_packing_amd as ibp

    dev = torch.device("cuda:0")
    say(f"workload {name}: generating")
    inst = workloads.generate(name)
    w = inst.w
    W, T, S = w.W, w.T, w.S
    flat = inst.data.reshape(-1)
    x = torch.from_numpy(flat.view(np.uint8)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    say(f"workload {name}: metadata")
    meta, counts = ibp.ibp_build_metadata(torch.from_numpy(inst.sample.reshape(-1).view(np.uint8)).to(dev), W, T)
    mask, bitval, c1 = oracle.build_meta(inst.sample.reshape(-1), W, T)
    assert counts == c1.tolist() and (meta.mask, meta.bitval) == (mask, bitval)

    say(f"workload {name}: compress {x.numel()} bytes")
    comp = ibp.ibp_compress(meta, x, S, err=err)
    off = comp.offsets.cpu().numpy().view(np.uint64)
    ref_off = oracle.offsets(flat, W, mask, bitval, S)
    assert np.array_equal(off, ref_off), "offset table differs"
    total = int(off[-1])
    stream_h = comp.stream[: (total + 7) // 8].cpu().numpy()
    nseg = off.size - 1
    rng = np.random.default_rng(7)
    ks = sorted(set([0, 1, nseg // 2, nseg - 2, nseg - 1] + rng.integers(0, nseg, 60).tolist()) - {-1})
    for k in ks:
        seg, nbits = oracle.encode_segment(flat, W, mask, bitval, S, k)
        assert nbits == int(off[k + 1] - off[k])
        want = np.unpackbits(seg, bitorder="little")[:nbits]
        assert np.array_equal(_bits(stream_h, int(off[k]), int(off[k + 1])), want), f"segment {k} differs"
    # bits of the last byte above the total are zero
    if total % 8:
        assert stream_h[-1] >> (total % 8) == 0

    say(f"workload {name}: decompress")
    out = ibp.ibp_decompress(meta, comp.stream, comp.offsets, comp.n_chunks, S, err=err)
    assert torch.equal(out, x), "round trip differs"
    del out

    if not w.gather:
        # the whole tensor from its stream in pinned host memory, read zero-copy
        say(f"workload {name}: decompress from the stream in pinned host memory")
        host = torch.zeros(ibp.ibp_stream_bytes(total), dtype=torch.uint8, pin_memory=True)
        host[: stream_h.size].copy_(torch.from_numpy(stream_h))
        out = ibp.ibp_decompress(meta, host, comp.offsets, comp.n_chunks, S, err=err)
        assert torch.equal(out, x), "round trip from pinned memory differs"
        del out, host

    if w.gather:
        say(f"workload {name}: gather from pinned host memory")
        n_rows = inst.data.shape[0]
        ids_np = workloads.gather_ids(name, n_rows, 1)[0]
        host = torch.empty((total + 7) // 8 + 16, dtype=torch.uint8, pin_memory=True)
        host[: stream_h.size].copy_(torch.from_numpy(stream_h))
        ids = torch.from_numpy(ids_np).to(dev)
        rows = ibp.ibp_decompress_gather(meta, host, comp.offsets, S, ids, err=err)
        got = rows.cpu().numpy().view(inst.data.dtype).reshape(len(ids_np), -1)
        assert np.array_equal(got, inst.data[ids_np])
        ref = oracle.decode_gather(stream_h, off, S, ids_np[:512], W, mask, bitval, inst.data.dtype)
        assert np.array_equal(got[:512].reshape(-1), ref)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("name", ["tiny", "gnn", "dlrm", "llm", "ids", "sparse", "llm16", "mixed"])
def test_workload_variants_full_size(name):
    """The variants bench.py also times, at the workloads' full sizes: the gather from
    the HBM-resident table, the fixed-slot table in pinned memory, position-dependent
    metadata, and (BF16 tensors) the ZipCCL exponent codec; sampled rows, segments
    and blocks against the oracle, everything else against the input."""
    import bit_packing_amd as ibp

    dev = torch.device("cuda:0")
    say(f"variants {name}: generating")
    inst = workloads.generate(name)
    w = inst.w
    W, T, S = w.W, w.T, w.S
    flat = inst.data.reshape(-1)
    x = torch.from_numpy(flat.view(np.uint8)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    rng = np.random.default_rng(11)
    sample = torch.from_numpy(inst.sample.reshape(-1).view(np.uint8)).to(dev)
    meta, _ = ibp.ibp_build_metadata(sample, W, T)

    if w.gather:
        n_rows = inst.data.shape[0]
        ids_np = workloads.gather_ids(name, n_rows, 1)[0]
        ids = torch.from_numpy(ids_np).to(dev)
        say(f"variants {name}: gather from the HBM-resident table")
        comp = ibp.ibp_compress(meta, x, S, err=err)
        rows = ibp.ibp_decompress_gather(meta, comp.stream, comp.offsets, S, ids, err=err)
        assert np.array_equal(rows.cpu().numpy().view(inst.data.dtype).reshape(len(ids_np), -1), inst.data[ids_np])
        del comp, rows
        say(f"variants {name}: fixed slots in pinned memory")
        row_bytes = inst.row_bytes
        slots = torch.empty(n_rows * row_bytes, dtype=torch.uint8, pin_memory=True)
        slots, flags = ibp.ibp_compress_slots(meta, x, S, slots=slots, err=err)
        torch.cuda.synchronize()
        got_flags = flags.cpu().numpy().view(np.uint64)
        picks = np.unique(np.concatenate([[0, n_rows - 1], rng.integers(0, n_rows, 40)]))
        for r in (int(v) for v in picks):
            ref_slot, ref_flag, used = oracle.encode_slots(inst.data[r], W, meta.mask, meta.bitval, S)
            assert ((int(got_flags[r // 64]) >> (r % 64)) & 1) == int(ref_flag[0]), f"flag of row {r}"
            nb = (int(used[0]) + 7) // 8
            got = slots[r * row_bytes: r * row_bytes + nb].numpy()
            assert np.array_equal(got, ref_slot[:nb]), f"slot {r}"
        out = ibp.ibp_decompress_gather_slots(meta, slots, flags, S, ids, err=err)
        assert np.array_equal(out.cpu().numpy().view(inst.data.dtype).reshape(len(ids_np), -1), inst.data[ids_np])
        del slots, out

    n_rows_sample = inst.sample.nbytes // (S * W // 8)
    if n_rows_sample:
        say(f"variants {name}: position-dependent metadata")
        srows = inst.sample.reshape(-1).view(np.uint8)[: n_rows_sample * S * W // 8]
        pmeta, counts = ibp.ibp_build_metadata_pos(torch.from_numpy(srows.copy()).to(dev), W, S, T)
        pm, pb, pc1 = oracle.build_meta_pos(srows, W, S, T)
        assert np.array_equal(pmeta.mask.cpu().numpy().view(np.uint64), pm)
        assert np.array_equal(pmeta.bitval.cpu().numpy().view(np.uint64), pb)
        assert np.array_equal(np.array(counts, np.uint64), pc1)
        pcomp = ibp.ibp_compress_pos(pmeta, x, err=err)
        off = pcomp.offsets.cpu().numpy().view(np.uint64)
        assert np.array_equal(off, oracle.offsets_pos(flat, W, pm, pb, S)), "position offsets"
        stream_h = pcomp.stream[: (int(off[-1]) + 7) // 8].cpu().numpy()
        nseg = off.size - 1
        cw = W // 8
        raw = flat.view(np.uint8)
        for k in sorted(set([0, nseg - 1] + rng.integers(0, nseg, 40).tolist())):
            seg_bytes = raw[k * S * cw: min((k + 1) * S, inst.n_chunks) * cw]
            seg, seg_off = oracle.encode_pos(seg_bytes, W, pm, pb, S)
            nbits = int(seg_off[-1])
            assert nbits == int(off[k + 1] - off[k])
            want = np.unpackbits(seg, bitorder="little")[:nbits]
            assert np.array_equal(_bits(stream_h, int(off[k]), int(off[k + 1])), want), f"segment {k}"
        out = ibp.ibp_decompress_pos(pmeta, pcomp.stream, pcomp.offsets, inst.n_chunks, err=err)
        assert torch.equal(out, x), "position round trip"
        del pcomp, out

    if w.dtype == "uint16" and w.sigma:
        say(f"variants {name}: ZipCCL exponent codec")
        table = ibp.ibp_zip_table_from_sigma(w.sigma)
        assert list(table) == oracle.zip_table(w.sigma).tolist()
        u = flat.view(np.uint16)
        z = ibp.ibp_zip_compress(table, x, err=err)
        eoff = z.eoff.cpu().numpy().view(np.uint64)
        nblk = eoff.size - 1
        sm_h, codes_h = z.sm.cpu().numpy(), z.codes.cpu().numpy()
        esc_h = z.esc[: int(eoff[-1])].cpu().numpy()
        for j in sorted(set([0, nblk - 1] + rng.integers(0, nblk, 40).tolist())):
            blk = u[j * 4096:(j + 1) * 4096]
            rsm, rcodes, resc, _ = oracle.zip_encode(blk, list(table))
            assert np.array_equal(sm_h[j * 4096: j * 4096 + blk.size], rsm), f"block {j} sign-mantissa"
            assert np.array_equal(codes_h[j * 1536:(j + 1) * 1536], rcodes), f"block {j} codes"
            assert np.array_equal(esc_h[int(eoff[j]):int(eoff[j + 1])], resc), f"block {j} escapes"
        back = ibp.ibp_zip_decompress(z, err=err)
        assert torch.equal(back.view(torch.uint8), x), "ZipCCL round trip"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("name", ["gnn", "llm"])
def test_compression_repeats_after_other_kernels(name):
    """The compressed stream does not depend on what ran before it: one full-size
    compression (single Mask and position metadata), then other codec kernels on the
    same GPU (decompression, gathers, fixed slots, the other compressor), then the
    same compression again; both results are compared byte for byte."""
    import bit_packing_amd as ibp

    dev = torch.device("cuda:0")
    say(f"repeat {name}: generating")
    inst = workloads.generate(name)
    w = inst.w
    W, T, S = w.W, w.T, w.S
    x = torch.from_numpy(inst.data.reshape(-1).view(np.uint8)).to(dev)
    sample = torch.from_numpy(inst.sample.reshape(-1).view(np.uint8)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    meta, _ = ibp.ibp_build_metadata(sample, W, T)
    nrs = inst.sample.nbytes // (S * W // 8)
    pmeta, _ = ibp.ibp_build_metadata_pos(sample[: nrs * S * W // 8], W, S, T, counts=False)

    def both():
        a = ibp.ibp_compress(meta, x, S, err=err)
        b = ibp.ibp_compress_pos(pmeta, x, err=err)
        torch.cuda.synchronize()
        out = []
        for c in (a, b):
            nb = (int(c.offsets[-1].item()) + 7) // 8
            out.append((c.offsets.cpu().numpy(), c.stream[:nb].cpu().numpy()))
        return out, a

    say(f"repeat {name}: first compression")
    first, comp = both()
    say(f"repeat {name}: other kernels")
    out = ibp.ibp_decompress(meta, comp.stream, comp.offsets, comp.n_chunks, S, err=err)
    assert torch.equal(out, x)
    del out
    if w.gather:
        ids = torch.from_numpy(workloads.gather_ids(name, inst.data.shape[0], 1)[0]).to(dev)
        ibp.ibp_decompress_gather(meta, comp.stream, comp.offsets, S, ids, err=err)
        slots, flags = ibp.ibp_compress_slots(meta, x, S, err=err)
        ibp.ibp_decompress_gather_slots(meta, slots, flags, S, ids, err=err)
        del slots, flags
    else:
        z = ibp.ibp_zip_compress(ibp.ibp_zip_table_from_sigma(w.sigma), x, err=err)
        ibp.ibp_zip_decompress(z, err=err)
        del z
    torch.cuda.synchronize()
    del comp
    say(f"repeat {name}: second compression")
    second, _ = both()
    assert int(err.item()) == 0
    for (o1, s1), (o2, s2), kind in zip(first, second, ("single Mask", "position metadata")):
        assert np.array_equal(o1, o2), f"{kind}: offsets differ between the two compressions"
        d = np.nonzero(s1 != s2)[0]
        assert d.size == 0, f"{kind}: {d.size} stream bytes differ, first at {d[:4]}"
