"""GPU parity of the comparison codec (BF16 exponent coding, the ZipCCL page's
section 2 A-B) against the oracle, bit-exact: sign-mantissa bytes, code planes,
escape exponents, escape offsets and round trips."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ibp():
    import bit_packing_amd

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bit_packing_amd.load_library()
    return bit_packing_amd


def say(msg):
    print(msg, flush=True)


def _bf16(rng, n, sigma, outliers=0.001):
    x = rng.standard_normal(n) * sigma
    hit = rng.random(n) < outliers
    x[hit] = rng.standard_normal(int(hit.sum()))
    f = x.astype(np.float32).view(np.uint32)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even


def _check(ibp, dev, u, table, tag):
    n = u.size
    x = torch.from_numpy(u.view(np.int16).copy()).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    z = ibp.ibp_zip_compress(bytes(table), x, err=err)
    sm, codes, esc, eoff = oracle.zip_encode(u, table)
    got_eoff = z.eoff.cpu().numpy().view(np.uint64)
    assert np.array_equal(got_eoff, eoff), f"{tag}: escape offsets"
    assert np.array_equal(z.sm[:n].cpu().numpy(), sm), f"{tag}: sign-mantissa bytes"
    assert np.array_equal(z.codes[:codes.size].cpu().numpy(), codes), f"{tag}: code planes"
    assert np.array_equal(z.esc[:esc.size].cpu().numpy(), esc), f"{tag}: escapes"
    out = ibp.ibp_zip_decompress(z, err=err)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), u), f"{tag}: round trip"
    torch.cuda.synchronize()
    assert int(err.item()) == 0


@pytest.mark.parametrize("sigma", [1e-3, 0.02, 1.0])
def test_zip_parity(ibp, sigma):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(int(sigma * 1e5))
    table = oracle.zip_table(sigma)
    for n in (1, 7, 8, 9, 4095, 4096, 4097, 2048 * 3 + 5, 3 * 4096 - 5, 4 * 4096, 4 * 4096 + 100, 100_003, (1 << 20) + 13):
        say(f"zip sigma={sigma} n={n}")
        _check(ibp, dev, _bf16(rng, n, sigma), table, f"n={n}")


def test_zip_every_bf16_pattern(ibp):
    """All 65,536 BF16 bit patterns (shuffled), so escapes of every exponent occur."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    u = np.concatenate([rng.permutation(65536), rng.permutation(65536)[:3001]]).astype(np.uint16)
    for table in (oracle.zip_table(1e-3), [0, 255, 1, 254, 127, 128, 126]):
        say(f"zip all patterns table={list(table)}")
        _check(ibp, dev, u, table, "all patterns")


def test_zip_corrupt_offsets_reported(ibp):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(6)
    u = _bf16(rng, 50_000, 1e-3, outliers=0.02)
    table = oracle.zip_table(1e-3)
    x = torch.from_numpy(u.view(np.int16).copy()).to(dev)
    z = ibp.ibp_zip_compress(bytes(table), x)
    z.eoff[4] += 1  # blocks 3 and 4 disagree with their codes
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.zeros(u.size, dtype=torch.int16, device=dev)
    ibp.ibp_zip_decompress(z, out=out, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & ibp.IBP_DEVERR_CORRUPT
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:3 * 4096], u[:3 * 4096]) and np.array_equal(got[5 * 4096:], u[5 * 4096:])
    assert not got[3 * 4096:5 * 4096].any()  # the two blocks were not decoded
