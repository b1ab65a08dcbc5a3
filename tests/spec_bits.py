"""Bit-string specification of Invariant Bit Packing, for tiny inputs only.

An implementation independent of the C oracle: a chunk is a Python string of
'0'/'1' characters, character b being bit b (least significant first), and every
step is done on strings -- no shifts, masks or popcounts.  It follows the IBP
technical summary (gist.science, paper 2605.30728), section "Algoritmo Core":
step 1 (metadata: positions whose value agrees on at least a fraction T of the
samples), step 2 (drop the invariant bits of matching chunks and flag every
chunk with a participation bit), step 3 (re-insert the invariant bits).  The
layout choices are the same readings the oracle states (header of participation
bits per segment, payloads after it, LSB-first stream).
"""
from __future__ import annotations

from fractions import Fraction


def int_to_bits(v: int, W: int) -> str:
    """W-character string, character b = bit b of v."""
    s = format(v, "b").rjust(W, "0")
    if len(s) != W:
        raise ValueError("value wider than W")
    return s[::-1]


def bits_to_int(s: str) -> int:
    return int(s[::-1], 2) if s else 0


def spec_meta(samples: list[str], T: float) -> tuple[str, str]:
    """(mask, bitval) strings from sample bit strings.

    Position b is invariant when its more frequent value occurs in at least a
    fraction Tppm/10^6 of the samples (Tppm = T rounded to parts per million).
    """
    N = len(samples)
    W = len(samples[0])
    frac = Fraction(round(T * 1_000_000), 1_000_000)
    mask, bitval = [], []
    for b in range(W):
        column = [s[b] for s in samples]
        ones = column.count("1")
        zeros = column.count("0")
        majority = max(ones, zeros)
        if Fraction(majority, N) >= frac:
            mask.append("1")
            bitval.append("1" if ones > zeros else "0")
        else:
            mask.append("0")
            bitval.append("0")
    return "".join(mask), "".join(bitval)


def _matches(chunk: str, mask: str, bitval: str) -> bool:
    return all(chunk[b] == bitval[b] for b in range(len(mask)) if mask[b] == "1")


def _free_bits(chunk: str, mask: str) -> str:
    return "".join(chunk[b] for b in range(len(mask)) if mask[b] == "0")


def spec_encode_bits(chunks: list[str], mask: str, bitval: str, S: int) -> tuple[str, list[int]]:
    """(stream as a bit string, bit offsets of the segments and the end)."""
    stream = ""
    offsets = [0]
    for start in range(0, len(chunks), S):
        seg = chunks[start:start + S]
        header = "".join("1" if _matches(c, mask, bitval) else "0" for c in seg)
        payload = "".join(_free_bits(c, mask) if _matches(c, mask, bitval) else c for c in seg)
        stream += header + payload
        offsets.append(len(stream))
    return stream, offsets


def bitstring_to_bytes(stream: str) -> bytes:
    padded = stream + "0" * (-len(stream) % 8)
    return bytes(bits_to_int(padded[i:i + 8]) for i in range(0, len(padded), 8))


def bytes_to_bitstring(data: bytes, nbits: int) -> str:
    return "".join(int_to_bits(x, 8) for x in data)[:nbits]


def spec_encode(values: list[int], W: int, mask: int, bitval: int, S: int) -> tuple[bytes, list[int]]:
    chunks = [int_to_bits(v, W) for v in values]
    stream, offsets = spec_encode_bits(chunks, int_to_bits(mask, W), int_to_bits(bitval, W), S)
    return bitstring_to_bytes(stream), offsets


def spec_decode(data: bytes, offsets: list[int], n: int, W: int, mask: int, bitval: int, S: int) -> list[int]:
    mask_s, bitval_s = int_to_bits(mask, W), int_to_bits(bitval, W)
    free = [b for b in range(W) if mask_s[b] == "0"]
    bits = bytes_to_bitstring(data, offsets[-1])
    out = []
    for k, start in enumerate(range(0, n, S)):
        m = min(S, n - start)
        seg = bits[offsets[k]:offsets[k + 1]]
        header, rest = seg[:m], seg[m:]
        for i in range(m):
            if header[i] == "1":
                payload, rest = rest[:len(free)], rest[len(free):]
                chunk = list(bitval_s)
                for t, b in enumerate(free):
                    chunk[b] = payload[t]
                out.append(bits_to_int("".join(chunk)))
            else:
                out.append(bits_to_int(rest[:W]))
                rest = rest[W:]
        if rest:
            raise ValueError("segment longer than its chunks")
    return out


# ------------------------------------------------------------------ position-dependent metadata
# Chunk i of every segment (row) has its own mask_i / bitval_i; the stream layout is unchanged.

def spec_meta_pos(rows: list[list[str]], T: float) -> list[tuple[str, str]]:
    """Per position i: spec_meta over the i-th chunk of every sample row."""
    S = len(rows[0])
    return [spec_meta([row[i] for row in rows], T) for i in range(S)]


def spec_encode_pos(values: list[int], W: int, masks: list[int], bitvals: list[int], S: int) -> tuple[bytes, list[int]]:
    chunks = [int_to_bits(v, W) for v in values]
    ms = [int_to_bits(m, W) for m in masks]
    bs = [int_to_bits(b, W) for b in bitvals]
    stream = ""
    offsets = [0]
    for start in range(0, len(chunks), S):
        seg = chunks[start:start + S]
        header = "".join("1" if _matches(c, ms[i], bs[i]) else "0" for i, c in enumerate(seg))
        payload = "".join(_free_bits(c, ms[i]) if _matches(c, ms[i], bs[i]) else c for i, c in enumerate(seg))
        stream += header + payload
        offsets.append(len(stream))
    return bitstring_to_bytes(stream), offsets
