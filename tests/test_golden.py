"""Oracle against hand-worked fixtures (tests/golden/*.txt).

The IBP page prints no worked example, so the fixtures were derived by hand from
its "Algoritmo Core" steps; each file carries its own derivation and citation.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _parse(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = (x.strip() for x in line.split("=", 1))
        out[key] = [float(t) if "." in t else int(t, 0) for t in val.split()]
    return out


@pytest.mark.parametrize("name", ["encode_w8_s4.txt", "encode_w8_s2.txt", "encode_w16_bytes.txt"])
def test_golden_encode(name):
    g = _parse(name)
    W, S, mask, bitval = g["W"][0], g["S"][0], g["mask"][0], g["bitval"][0]
    if "values" in g:
        x = np.array(g["values"], np.uint64)
        n = x.size
    else:
        x = np.array(g["bytes"], np.uint8)
        n = x.size // (W // 8)
    stream, off = oracle.encode(x, W, mask, bitval, S)
    assert off.tolist() == g["offsets"]
    assert stream.tolist() == g["stream"]
    back = oracle.decode(stream, off, n, W, mask, bitval, S,
                         out_dtype=None if "values" in g else np.uint8)
    assert back.tolist() == x.tolist()


def test_golden_meta():
    g = _parse("meta_w4.txt")
    W = g["W"][0]
    x = np.array(g["samples"], np.uint64)
    for tk, mk, bk in (("T", "mask", "bitval"), ("T2", "mask2", "bitval2"), ("T3", "mask3", "bitval3")):
        mask, bitval, counts = oracle.build_meta(x, W, g[tk][0])
        assert counts.tolist() == g["counts"]
        assert (mask, bitval) == (g[mk][0], g[bk][0]), tk


def test_golden_slots():
    g = _parse("slots_w8_s4.txt")
    W, S, mask, bitval = g["W"][0], g["S"][0], g["mask"][0], g["bitval"][0]
    x = np.array(g["bytes"], np.uint8)
    slots, flags, used = oracle.encode_slots(x, W, mask, bitval, S)
    assert slots.tolist() == g["slots"]
    assert flags.tolist() == g["flags"]
    assert used.tolist() == g["used_bits"]
    back = oracle.decode_slots_gather(slots, flags, S, np.array([1, 0, 1], np.int64), W, mask, bitval)
    assert back.tolist() == g["bytes"][4:] + g["bytes"][:4] + g["bytes"][4:]


def test_golden_encode_pos():
    g = _parse("encode_pos_w4_s2.txt")
    W, S = g["W"][0], g["S"][0]
    x = np.array(g["values"], np.uint64)
    stream, off = oracle.encode_pos(x, W, g["mask"], g["bitval"], S)
    assert off.tolist() == g["offsets"]
    assert stream.tolist() == g["stream"]
    assert oracle.decode_pos(stream, off, x.size, W, g["mask"], g["bitval"], S).tolist() == x.tolist()


def test_golden_zip():
    g = _parse("zip_bf16.txt")
    x = np.array(g["values"], np.uint16)
    sm, codes, esc, eoff = oracle.zip_encode(x, g["table"])
    assert sm.tolist() == g["sm"]
    assert codes.size == 1536
    assert (codes[0], codes[512], codes[1024]) == (g["plane0"][0], g["plane1"][0], g["plane2"][0])
    assert not codes[1:512].any() and not codes[513:1024].any() and not codes[1025:].any()
    assert esc.tolist() == g["esc"] and eoff.tolist() == g["eoff"]
    assert oracle.zip_decode(sm, codes, esc, eoff, x.size, g["table"]).tolist() == g["values"]
