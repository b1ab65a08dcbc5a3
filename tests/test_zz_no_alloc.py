"""ibp_compress_noalloc (the compression entry point that allocates nothing; its
workspace is a fixed device array inside the library) against ibp_compress, bit for
bit, through the C ABI: two calls in a row, the second with a smaller input, so the
second call runs on the array the first one left behind."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


def _data(rng, n, W, mask, bitval, p_match):
    t = {16: np.uint16, 32: np.uint32, 64: np.uint64}[W]
    v = rng.integers(0, 1 << 62, size=n, dtype=np.uint64) * np.uint64(4) + rng.integers(0, 4, size=n, dtype=np.uint64)
    v = (v & np.uint64((1 << W) - 1)).astype(t)
    keep = rng.random(n) < p_match
    v[keep] = (v[keep] & t(~mask & ((1 << W) - 1))) | t(bitval)
    return v


def _noalloc(ibp, meta, x, S, out_stream, out_off, err):
    lib = ibp.load_library()
    return lib.ibp_compress_noalloc(ctypes.byref(meta), x.data_ptr(), x.numel() * x.element_size(), S,
                                    out_stream.data_ptr(), out_stream.numel(), out_off.data_ptr(), err.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("W,S,mask,bitval", [(64, 256, 0xFFFFFFFFFF000000, 0), (32, 128, 0xC0000000, 0),
                                             (16, 1024, 0x7C00, 0x3800), (32, 100, 0x78000000, 0x38000000)])
def test_noalloc_matches_compress(ibp, W, S, mask, bitval):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(W * 31 + S)
    meta = ibp.make_meta(W, mask, bitval)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for n in (3_000_001, 250_003):  # the second call smaller than the first
        print(f"no-alloc compress: W={W} S={S} n={n}", flush=True)
        v = _data(rng, n, W, mask, bitval, 0.95)
        x = torch.from_numpy(v.view(np.uint8).copy()).to(dev)
        ref = ibp.ibp_compress(meta, x, S, err=err)
        cap = ibp.ibp_max_stream_bytes(n, W)
        out_stream = torch.full((cap,), 0x5A, dtype=torch.uint8, device=dev)
        out_off = torch.full((ibp.ibp_num_segments(n, S) + 1,), -7, dtype=torch.int64, device=dev)
        assert _noalloc(ibp, meta, x, S, out_stream, out_off, err) == ibp.IBP_OK
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out_off, ref.offsets), "offsets differ from ibp_compress"
        nb = (int(ref.offsets[-1].item()) + 7) // 8
        assert torch.equal(out_stream[:nb], ref.stream[:nb]), "stream differs from ibp_compress"

